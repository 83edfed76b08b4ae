"""All-position logits in prefill and the device-resident greedy loop.

all_logits (rml "The decoder", section "One forward pass", step 7: only the
rows that need logits get the final norm and output product, the last or all)
is compared row by row with the oracle's prefill over every row.  The device
loop (Pantheon, section "Optional GPU Paths": the whole layer chain on the
device, tokens never crossing to the host between steps) must give exactly the
tokens and logits of the host-driven loop (dec_decode then dec_greedy each
step), and every token it chose must be the oracle's greedy choice (within the
tie margin) when the oracle is fed the loop's own tokens.
"""
import numpy as np
import pytest
import torch

from decoder_only_forward_amd import configs, synth
from parity_util import Pair, check_argmax, check_logits

pytestmark = pytest.mark.gpu


def _all_rows(pair, prompt, what, start_pos=0, seq=0):
    g = pair.gpu.prefill(prompt, seq=seq, start_pos=start_pos, all_logits=True).cpu().numpy()
    r = pair.ora.prefill(prompt, slot=seq, start_pos=start_pos, rows=list(range(len(prompt))))
    assert g.shape == r["logits"].shape == (len(prompt), pair.cfg.vocab)
    for t in range(len(prompt)):
        check_logits(g[t], r["logits"][t], f"{what} row {t}", **pair.tol)
        check_argmax(g[t], r["logits"][t], f"{what} row {t}", **pair.tol)
    return g


@pytest.mark.parametrize("cfg", [configs.TINY, configs.TINY_BF16, configs.TINY_MOE, configs.TINY_KVBF16],
                         ids=lambda c: c.name)
def test_all_logits_prefill_tiny(cfg):
    """8 rows: the LM head as a GEMV over 8 rows (fp32 weights: the fp32 GEMM
    writing straight into the caller's buffer)."""
    pair = Pair(cfg, max_prefill=8)
    prompt = synth.tokens(0, synth.PROMPT_STREAM, 8, cfg.vocab).tolist()
    _all_rows(pair, prompt, cfg.name)
    assert pair.gpu.length(0) == 8


def test_all_logits_prefill_smollm2_128_rows():
    """128 rows: the LM head runs as the MFMA GEMM into the caller's buffer."""
    cfg = configs.SMOLLM2
    pair = Pair(cfg, max_prefill=128)
    prompt = synth.tokens(0, synth.PROMPT_STREAM, 128, cfg.vocab).tolist()
    g = _all_rows(pair, prompt, "smollm2")
    # the last row is what the last-row-only prefill returns
    other = Pair(cfg, max_prefill=128, weights=pair.w)
    last = other.gpu.prefill(prompt).cpu().numpy()
    check_logits(g[-1], last, "last row vs last-row prefill")


def test_all_logits_append_and_ring_wrap():
    """AppendPrefill (start_pos > 0), and a prefill that wraps the ring inside
    one call (position-by-position path, one logits row per position)."""
    cfg = configs.TINY_BF16
    pair = Pair(cfg, max_prefill=8)
    toks = synth.tokens(0, synth.PROMPT_STREAM, 14, cfg.vocab).tolist()
    _all_rows(pair, toks[:6], "first chunk")
    _all_rows(pair, toks[6:], "appended chunk", start_pos=6)
    cfg = configs.TINY_WINDOW
    pair = Pair(cfg, max_prefill=16)
    _all_rows(pair, synth.tokens(0, synth.PROMPT_STREAM, 16, cfg.vocab).tolist(), "ring wrap")


def _host_loop(model, tokens, steps, B):
    tok = np.asarray(tokens, dtype=np.int32)
    out = []
    lg = torch.empty((B, model.cfg.vocab), device="cuda")
    for _ in range(steps):
        pos = [model.length(b) for b in range(B)]
        model.decode(tok, pos, logits=lg)
        tok = model.greedy(lg, B)
        out.append(tok.copy())
    return np.stack(out), lg.cpu().numpy()


def _prefilled_pair(cfg, B, P, max_prefill=None, weights=None):
    pair = Pair(cfg, n_slots=B, max_prefill=max_prefill or P, weights=weights)
    pr = synth.prompts(cfg, B, P)
    first = []
    for b in range(B):
        lg = pair.gpu.prefill(pr[b].tolist(), seq=b)
        first.append(int(torch.argmax(lg).item()))
    return pair, pr, first


@pytest.mark.parametrize("cfg,B,P,steps", [(configs.TINY_BF16, 3, 5, 9), (configs.TINY_MOE, 2, 4, 6),
                                           (configs.TINY_WINDOW, 2, 3, 9), (configs.SMOLLM2, 32, 4, 5)],
                         ids=["tiny-bf16", "tiny-moe", "tiny-window-wrap", "smollm2-b32"])
def test_device_loop_equals_host_loop(cfg, B, P, steps):
    """Same tokens and the same final logits, bit for bit, as the host-driven
    loop; the device loop replays one captured graph per step."""
    a, _, first = _prefilled_pair(cfg, B, P)
    b, _, first_b = _prefilled_pair(cfg, B, P, weights=a.w)
    assert first == first_b
    n0 = a.gpu.graph_count()
    choices, lg = a.gpu.decode_greedy(first, steps)
    torch.cuda.synchronize()
    want, want_lg = _host_loop(b.gpu, first, steps, B)
    np.testing.assert_array_equal(choices.cpu().numpy(), want)
    np.testing.assert_array_equal(lg.cpu().numpy(), want_lg)
    assert all(a.gpu.length(r) == P + steps for r in range(B))
    assert a.gpu.graph_count() > n0


@pytest.mark.parametrize("cfg", [configs.TINY, configs.TINY_BF16, configs.TINY_KVBF16], ids=lambda c: c.name)
def test_device_loop_tokens_are_the_oracles_greedy_choices(cfg):
    B, P, steps = 2, 6, 8
    pair, pr, first = _prefilled_pair(cfg, B, P)
    for b in range(B):
        pair.ora.prefill(pr[b].tolist(), slot=b)
    choices, lg = pair.gpu.decode_greedy(first, steps)
    choices = choices.cpu().numpy()
    lg = lg.cpu().numpy()
    inp = np.asarray(first)
    for s in range(steps):
        r = pair.ora.decode(inp.tolist(), [P + s] * B)
        for b in range(B):
            # the loop's choice at step s from its own logits must be the oracle's
            # greedy choice for the same inputs (within the tie margin)
            onehot = np.full(cfg.vocab, -1.0)
            onehot[choices[s, b]] = 1.0
            check_argmax(onehot, r["logits"][b], f"{cfg.name} step {s} row {b}", **pair.tol)
        if s == steps - 1:
            for b in range(B):
                check_logits(lg[b], r["logits"][b], f"{cfg.name} last-step logits row {b}", **pair.tol)
        inp = choices[s]
