"""Prefill into a ring cache past its size, in one pass (deferred commit).

A chunk whose positions run past the ring's max_seq slots would overwrite
slots that its own earlier queries still read.  The library holds the chunk's
K/V back until the chunk's attention is done, reading history from the ring
and the chunk from its buffer, each query limited to its window
[p - W + 1, p] (rml "The decoder", section "Attend"), and then commits the
last min(n, W) rows (zLLM "The Algorithm Layer", section 5: AppendPrefill
appends a span after existing history).  The oracle stores and attends
position by position, which is the plain definition.
"""
import numpy as np
import pytest
import torch

from decoder_only_forward_amd import configs, synth
from oracle import oracle as O
from parity_util import Pair, check_argmax, check_hidden, check_logits, oracle_kind, rel_l2, tol
from test_gpu_fullwidth import _host

pytestmark = pytest.mark.gpu


def _chunks(pair, toks, sizes, what):
    """Prefill toks in chunks of the given sizes; every row's logits and every
    layer's hidden state against the oracle."""
    start = 0
    for n in sizes:
        chunk = toks[start:start + n]
        hid, _, _ = pair.capture_buffers(n)
        g = pair.gpu.prefill(chunk, start_pos=start, all_logits=True).cpu().numpy()
        r = pair.ora.prefill(chunk, start_pos=start, rows=list(range(n)), capture=True)
        for t in range(n):
            check_logits(g[t], r["logits"][t], f"{what} chunk@{start} row {t}", **pair.tol)
            check_argmax(g[t], r["logits"][t], f"{what} chunk@{start} row {t}", **pair.tol)
        check_hidden(hid.cpu().numpy(), r["hidden"], f"{what} chunk@{start}", **pair.tol)
        start += n
        assert pair.gpu.length(0) == start
    pair.gpu.set_capture(None, None, None)
    return start


@pytest.mark.parametrize("cfg", [configs.TINY_WINDOW,
                                 configs.TINY_WINDOW.replace(name="tiny-window-bf16w", weight_dtype=0, ffn_dim=192),
                                 configs.TINY_WINDOW.replace(name="tiny-window-moe", n_experts=8, top_k=2),
                                 configs.TINY_WINDOW.replace(name="tiny-window-kvbf16", kv_bf16=True),
                                 configs.TINY_WINDOW.replace(name="tiny-window-kvf24", kv_f24=True)],
                         ids=lambda c: c.name)
def test_tiny_ring_appends_past_the_ring(cfg):
    """W = 5: chunks of 3, 4 (wraps), 9 (longer than the ring), 1, then decode."""
    pair = Pair(cfg, max_prefill=9)
    toks = synth.tokens(0, synth.PROMPT_STREAM, 17, cfg.vocab).tolist()
    n = _chunks(pair, toks, [3, 4, 9, 1], cfg.name)
    nxt = 7
    for s in range(4):
        g = pair.gpu.decode([nxt], [n + s]).cpu().numpy()
        r = pair.ora.decode([nxt], [n + s])
        check_logits(g[0], r["logits"][0], f"{cfg.name} decode {s}", **pair.tol)
        nxt = int(np.argmax(r["logits"][0]))


def test_smollm2_width_ring_at_full_depth():
    """SmolLM2 shape with a 64-slot window (head_dim 64, 3 query heads per kv
    head: the MFMA prefill kernel with window masking and deferred commit)."""
    cfg = configs.SMOLLM2.replace(name="smollm2-w64", sliding_window=64, max_seq=64)
    pair = Pair(cfg, max_prefill=100)
    toks = synth.tokens(0, synth.PROMPT_STREAM, 200, cfg.vocab).tolist()
    _chunks(pair, toks, [40, 50, 100, 10], "smollm2-w64")


def test_smollm2_width_ring_at_full_depth_f24_cache():
    """The same appends with a 24-bit cache: the general MFMA prefill kernel
    reads ring slots and chunk rows in that format, the commit copies them."""
    cfg = configs.SMOLLM2.replace(name="smollm2-w64-kvf24", sliding_window=64, max_seq=64, kv_f24=True)
    pair = Pair(cfg, max_prefill=100)
    toks = synth.tokens(0, synth.PROMPT_STREAM, 200, cfg.vocab).tolist()
    _chunks(pair, toks, [40, 50, 100, 10], "smollm2-w64-kvf24")


def _mistral_ring(P0, n, sample, kv_bf16=False):
    """Full-width one-layer Mistral-7B: prefill P0 tokens, then append n more
    in one call (deferred commit); sampled rows of the appended chunk, and one
    decode step after it, against the oracle."""
    cfg = configs.one_layer(configs.MISTRAL)
    if kv_bf16:
        cfg = cfg.replace(name=cfg.name + "-kvbf16", kv_bf16=True)
    torch.manual_seed(0)
    wd = synth.make_weights(cfg, seed=0, device="cuda")
    w = _host(wd)
    from decoder_only_forward_amd.dec import DecModel
    gpu = DecModel(cfg, wd, max_batch=1, max_prefill=max(P0, n) if P0 else n)
    toks = synth.prompts(cfg, 1, P0 + n)[0].tolist()
    if P0:
        gpu.prefill(toks[:P0])
    hid = torch.full((2, n, cfg.hidden), float("nan"), device="cuda")
    gpu.set_capture(hid, None, None)
    lg = gpu.prefill(toks[P0:], start_pos=P0, all_logits=True).cpu().numpy()
    gpu.set_capture(None, None, None)
    nxt = int(np.argmax(lg[-1]))
    dl = gpu.decode([nxt], [P0 + n]).cpu().numpy()[0]
    torch.cuda.synchronize()
    hid = hid.cpu().numpy()
    ora = O.OracleModel(cfg, w, n_slots=1, max_seq=cfg.max_seq, kind=oracle_kind(cfg))
    rows = [P0 + t for t in sample] + [P0 + n]
    r = ora.prefill(toks + [nxt], rows=rows, partial=True, capture=True)
    tl = tol(cfg)
    for i, t in enumerate(sample):
        rl = rel_l2(hid[1, t], r["hidden"][1, P0 + t])
        assert rl <= tl["rel"], f"row {P0 + t}: hidden rel L2 {rl:.3e}"
        check_logits(lg[t], r["logits"][i], f"appended row {P0 + t}", **tl)
        check_argmax(lg[t], r["logits"][i], f"appended row {P0 + t}", **tl)
    check_logits(dl, r["logits"][-1], "decode after the append", **tl)
    assert gpu.length(0) == P0 + n + 1
    gpu.close()


def test_mistral_one_layer_append_512_after_a_full_ring():
    _mistral_ring(4096, 512, [0, 1, 255, 511])


def test_mistral_one_layer_single_prefill_longer_than_the_ring():
    _mistral_ring(0, 4396, [0, 4095, 4096, 4200, 4395])


@pytest.mark.parametrize("kv_bf16", [False, True], ids=["f32-cache", "bf16-cache"])
def test_mistral_one_layer_decode_whose_new_slot_is_in_a_middle_split(kv_bf16):
    """After 6096 positions the ring's next slot is 2000: the B = 1 decode
    attention runs 32 splits of 128 slots, and split 15, not the first or the
    last, stores the new key/value before reading its range."""
    _mistral_ring(4096, 2000, [0, 1999], kv_bf16=kv_bf16)
