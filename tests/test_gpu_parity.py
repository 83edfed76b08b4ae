"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Decode is teacher-forced by the oracle's own greedy stream: both sides read
the same tokens, so a legitimately tied step cannot derail the comparison.
Full-depth models are compared on every logit and every layer's hidden state;
full-width one-layer models (every kernel at its real size) on sampled rows.
"""
import numpy as np
import pytest
import torch

from decoder_only_forward_amd import configs, synth
from oracle import oracle as O
from parity_util import (Pair, check_argmax, check_experts, check_hidden, check_logits)

pytestmark = pytest.mark.gpu


def _run_stream(pair, prompt, steps, what, slot=0):
    """Prefill `prompt` into slot 0, then `steps` greedy decode steps (B=1),
    comparing logits, argmax, hidden states and expert ids at every call."""
    c = pair.cfg
    n = len(prompt)
    hid, ids, rl = pair.capture_buffers(n)
    g = pair.gpu.prefill(prompt)
    r = pair.ora.prefill(prompt, capture=True)
    torch.cuda.synchronize()
    check_logits(g.cpu().numpy(), r["logits"][0], f"{what} prefill", **pair.tol)
    check_argmax(g.cpu().numpy(), r["logits"][0], f"{what} prefill", **pair.tol)
    check_hidden(hid.cpu().numpy(), r["hidden"], f"{what} prefill", **pair.tol)
    if c.n_experts:
        check_experts(ids.cpu().numpy(), r["ids"], r["router"], c.top_k, f"{what} prefill")
    nxt = int(np.argmax(r["logits"][0]))
    for s in range(steps):
        p = n + s
        hid, ids, rl = pair.capture_buffers(1)
        g = pair.gpu.decode([nxt], [p])
        r = pair.ora.decode([nxt], [p], capture=True)
        torch.cuda.synchronize()
        check_logits(g.cpu().numpy()[0], r["logits"][0], f"{what} step {s}", **pair.tol)
        check_argmax(g.cpu().numpy()[0], r["logits"][0], f"{what} step {s}", **pair.tol)
        check_hidden(hid.cpu().numpy(), r["hidden"], f"{what} step {s}", **pair.tol)
        if c.n_experts:
            check_experts(ids.cpu().numpy(), r["ids"], r["router"], c.top_k, f"{what} step {s}")
        nxt = int(np.argmax(r["logits"][0]))
    assert pair.gpu.length(0) == pair.ora.length(0) == n + steps


TINY_SET = [configs.TINY, configs.TINY_MOE, configs.TINY_BIAS, configs.TINY_BF16,
            configs.TINY_BF16.replace(name="tiny-bf16-moe", n_experts=8, top_k=2),
            configs.TINY_LLAMA3, configs.TINY_HALF,
            configs.TINY_BF16.replace(name="tiny-bf16-llama3-half", rope_pairing=1, rope_scaling=1,
                                      rope_orig_ctx=64)]


@pytest.mark.parametrize("cfg", TINY_SET, ids=lambda c: c.name)
def test_tiny_prefill_then_greedy_decode(cfg):
    """The tiny workload: 8 prompt tokens at start_pos 0, then 8 greedy steps."""
    pair = Pair(cfg, max_prefill=8)
    prompt = synth.tokens(0, synth.PROMPT_STREAM, 8, cfg.vocab).tolist()
    _run_stream(pair, prompt, 8, cfg.name)


def test_tiny_window_ring_wraps_in_decode_and_prefill():
    cfg = configs.TINY_WINDOW          # W = 5 ring
    prompt = synth.tokens(0, synth.PROMPT_STREAM, 4, cfg.vocab).tolist()
    _run_stream(Pair(cfg, max_prefill=16), prompt, 11, "ring decode")
    # a 16-token prefill wraps the ring inside one call (position-by-position path)
    prompt = synth.tokens(0, synth.PROMPT_STREAM, 16, cfg.vocab).tolist()
    _run_stream(Pair(cfg, max_prefill=16), prompt, 3, "ring prefill")


@pytest.mark.parametrize("cfg", [configs.TINY, configs.TINY_BF16, configs.TINY_MOE], ids=lambda c: c.name)
def test_tiny_batched_decode_rows_are_independent(cfg):
    B, P = 3, 5
    pair = Pair(cfg, n_slots=B, max_prefill=P)
    pr = synth.prompts(cfg, B, P)
    nxt = []
    for b in range(B):
        pair.gpu.prefill(pr[b].tolist(), seq=b)
        r = pair.ora.prefill(pr[b].tolist(), slot=b)
        nxt.append(int(np.argmax(r["logits"][0])))
    for s in range(4):
        pos = [P + s] * B
        hid, _, _ = pair.capture_buffers(B)
        g = pair.gpu.decode(nxt, pos).cpu().numpy()
        r = pair.ora.decode(nxt, pos, capture=True)
        for b in range(B):
            check_logits(g[b], r["logits"][b], f"row {b} step {s}")
            check_argmax(g[b], r["logits"][b], f"row {b} step {s}")
        check_hidden(hid.cpu().numpy(), r["hidden"], f"step {s}")
        nxt = [int(np.argmax(r["logits"][b])) for b in range(B)]


def test_append_prefill_continues_a_sequence():
    """AppendPrefill (start_pos > 0) attends to the cached history."""
    cfg = configs.TINY_BF16
    pair = Pair(cfg, max_prefill=8)
    toks = synth.tokens(0, synth.PROMPT_STREAM, 14, cfg.vocab).tolist()
    pair.gpu.prefill(toks[:6])
    pair.ora.prefill(toks[:6])
    hid, _, _ = pair.capture_buffers(8)
    g = pair.gpu.prefill(toks[6:], start_pos=6)
    r = pair.ora.prefill(toks[6:], start_pos=6, capture=True)
    check_logits(g.cpu().numpy(), r["logits"][0], "append")
    check_hidden(hid.cpu().numpy(), r["hidden"], "append")


def test_gpu_is_deterministic():
    cfg = configs.TINY_BF16
    prompt = synth.tokens(0, synth.PROMPT_STREAM, 8, cfg.vocab).tolist()
    outs = []
    for _ in range(2):
        pair = Pair(cfg, max_prefill=8)
        a = pair.gpu.prefill(prompt).cpu().numpy()
        b = pair.gpu.decode([3], [8]).cpu().numpy()
        outs.append((a, b))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


def test_smollm2_prefill_128_and_decode_b1():
    """SmolLM2-135M shape at full depth: P = 128, then greedy decode at B = 1."""
    cfg = configs.SMOLLM2
    pair = Pair(cfg, max_prefill=128)
    prompt = synth.tokens(0, synth.PROMPT_STREAM, 128, cfg.vocab).tolist()
    _run_stream(pair, prompt, 4, "smollm2")


def test_smollm2_decode_b32():
    """Batch-32 decode at full depth (short prompts keep the oracle fast)."""
    cfg = configs.SMOLLM2
    B, P = 32, 4
    pair = Pair(cfg, n_slots=B, max_prefill=P)
    pr = synth.prompts(cfg, B, P)
    nxt = []
    for b in range(B):
        pair.gpu.prefill(pr[b].tolist(), seq=b)
        r = pair.ora.prefill(pr[b].tolist(), slot=b)
        nxt.append(int(np.argmax(r["logits"][0])))
    for s in range(2):
        pos = [P + s] * B
        g = pair.gpu.decode(nxt, pos).cpu().numpy()
        r = pair.ora.decode(nxt, pos)
        for b in range(B):
            check_logits(g[b], r["logits"][b], f"row {b} step {s}")
            check_argmax(g[b], r["logits"][b], f"row {b} step {s}")
        nxt = [int(np.argmax(r["logits"][b])) for b in range(B)]


def test_smollm2_decode_b32_after_prompt_128():
    """The SmolLM2 workload's batch-32 decode at positions 128..255: 32 rows
    each after a 128-token prompt, teacher-forced.  Every row is compared with
    the oracle at the first two steps; rows 0, 15 and 31 at sampled steps up
    to position 255 (the oracle recomputes a row as one prefill over its
    prompt and teacher tokens, equal to per-token calls)."""
    cfg = configs.SMOLLM2
    B, P, steps = 32, 128, 128
    pair = Pair(cfg, n_slots=B, max_prefill=P)
    pr = synth.prompts(cfg, B, P)
    teach = synth.prompts(cfg, B, steps, stream=synth.TEACHER_STREAM)
    for b in range(B):
        pair.gpu.prefill(pr[b].tolist(), seq=b)
    lg = torch.empty((B, cfg.vocab), device="cuda")
    sampled = {0: None, 1: None, 64: None, 127: None}
    for s in range(steps):
        pair.gpu.decode(teach[:, s].tolist(), [P + s] * B, logits=lg)
        if s in sampled:
            sampled[s] = lg.cpu().numpy()
    for b in range(B):
        long_row = b in (0, 15, 31)
        st = sorted(sampled) if long_row else [0, 1]
        seq = pr[b].tolist() + teach[b, :st[-1] + 1].tolist()
        ora = O.OracleModel(cfg, pair.w, n_slots=1, max_seq=cfg.max_seq)
        r = ora.prefill(seq, rows=[P + s for s in st], partial=True)
        for i, s in enumerate(st):
            check_logits(sampled[s][b], r["logits"][i], f"row {b} step {s}")
            check_argmax(sampled[s][b], r["logits"][i], f"row {b} step {s}")


def test_decode_graph_replay_is_bit_identical_to_eager():
    """Decode steps replayed from a captured HIP graph give exactly the logits of
    eager launches (the capture of test hidden states forces the eager path)."""
    cfg = configs.SMOLLM2
    B, P = 4, 6
    w = synth.make_weights(cfg)
    from parity_util import to_device
    from decoder_only_forward_amd.dec import DecModel
    wd = to_device(w)
    pr = synth.prompts(cfg, B, P)
    teach = synth.prompts(cfg, B, 5, stream=synth.TEACHER_STREAM)
    outs = []
    for eager in (True, False):
        m = DecModel(cfg, wd, max_batch=B, max_prefill=P)
        for b in range(B):
            m.prefill(pr[b].tolist(), seq=b)
        if eager:  # capture buffers hold B rows: set after the P-row prefills
            hid = torch.empty((cfg.n_layers + 1, B, cfg.hidden), device="cuda")
            m.set_capture(hid)
        lg = torch.empty((B, cfg.vocab), device="cuda")
        steps = []
        for s in range(5):
            m.decode(teach[:, s].tolist(), [P + s] * B, logits=lg)
            steps.append(lg.cpu().numpy().copy())
        outs.append(steps)
        if not eager:
            assert m.graph_count() >= 1
        m.close()
    for s in range(5):
        assert np.array_equal(outs[0][s], outs[1][s]), f"step {s}"
