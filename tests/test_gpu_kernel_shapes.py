"""Parity at shapes chosen to reach the edges of the prefill kernels.

* The 256 x 256-tile GEMM (taken when a projection has at least one tile per
  CU) with a feature count that is not a multiple of 256 and a token count that
  is not a multiple of 256: the clamped loads and masked stores of both tails.
* The tile-image prefill attention with ragged chunk lengths and start_pos > 0
  (AppendPrefill reading the cached history through the per-layer tile pass),
  with an fp32 and with a bf16 K/V cache, at head_dim 64 and 128.

Each case compares every prefill row's hidden state after the layer and the
last row's logits with the oracle.
"""
import numpy as np
import pytest
import torch

from decoder_only_forward_amd import configs, synth
from parity_util import Pair, check_argmax, check_experts, check_hidden, check_logits, rel_l2, tol, HIDDEN_REL_L2

pytestmark = pytest.mark.gpu


def _chunks(pair, toks, sizes, what):
    c = pair.cfg
    tl = pair.tol
    hid_tol = HIDDEN_REL_L2 if not c.kv_bf16 else tl["rel"]
    start = 0
    for n in sizes:
        part = toks[start:start + n]
        hid, _, _ = pair.capture_buffers(n)
        g = pair.gpu.prefill(part, start_pos=start).cpu().numpy()
        r = pair.ora.prefill(part, start_pos=start, capture=True)
        torch.cuda.synchronize()
        h = hid.cpu().numpy()
        for t in range(n):
            rl = rel_l2(h[1, t], r["hidden"][1, t])
            assert rl <= hid_tol, f"{what} chunk at {start}: row {t} hidden rel L2 {rl:.3e}"
        check_logits(g, r["logits"][0], f"{what} chunk at {start}", **tl)
        check_argmax(g, r["logits"][0], f"{what} chunk at {start}", **tl)
        start += n


ODD = configs.ModelConfig("odd-1l", n_layers=1, hidden=512, n_heads=4, n_kv_heads=2, head_dim=128,
                          ffn_dim=14400, vocab=1000, max_seq=1024, rms_eps=1e-5, rope_theta=1e4)


def test_gemm_feature_and_token_tails_on_the_large_tile_kernel():
    """gate|up has 28800 features (112.5 tiles of 256) and the prompt 700 tokens
    (2.7 tiles): 339 tiles, so the 256x256 kernel runs with both tails."""
    pair = Pair(ODD, max_prefill=700)
    toks = synth.tokens(0, synth.PROMPT_STREAM, 700, ODD.vocab).tolist()
    _chunks(pair, toks, [700], "odd shape")


@pytest.mark.parametrize("kv_bf16", [False, True], ids=["fp32-cache", "bf16-cache"])
@pytest.mark.parametrize("base", [configs.SMOLLM2, configs.MISTRAL], ids=["hd64-g3", "hd128-g4"])
def test_tile_attention_appends_ragged_chunks(base, kv_bf16):
    """Chunks of 100, 93 and 57 tokens (starts 0, 100, 193): every chunk after
    the first reads history written by earlier calls through the tile pass."""
    cfg = configs.one_layer(base).replace(name=base.name + "-1l-append", kv_bf16=kv_bf16,
                                          sliding_window=0, max_seq=256)
    pair = Pair(cfg, max_prefill=100)
    toks = synth.tokens(0, synth.PROMPT_STREAM, 250, cfg.vocab).tolist()
    _chunks(pair, toks, [100, 93, 57], cfg.name)


def test_fused_swiglu_decode_projection_at_prefill_and_decode_rows():
    """gate|up of 2 x 14400 features is 225 row tiles, so the decode projection
    takes one k split and writes silu(gate) * up from its epilogue: a 40-token
    prefill (40 rows, the 8-tile kernel) into each of 3 slots, then 2 decode
    steps at B = 3 (the 2-tile kernel with spare columns), every row's hidden
    state after the layer and the logits against the oracle."""
    B, P = 3, 40
    pair = Pair(ODD, n_slots=B, max_prefill=P)
    c, tl = ODD, pair.tol
    prompts = synth.prompts(c, B, P)
    for b in range(B):
        hid, _, _ = pair.capture_buffers(P)
        g = pair.gpu.prefill(prompts[b].tolist(), seq=b).cpu().numpy()
        r = pair.ora.prefill(prompts[b].tolist(), slot=b, capture=True)
        torch.cuda.synchronize()
        h = hid.cpu().numpy()
        for t in range(P):
            rl = rel_l2(h[1, t], r["hidden"][1, t])
            assert rl <= HIDDEN_REL_L2, f"prefill slot {b}: row {t} hidden rel L2 {rl:.3e}"
        check_logits(g, r["logits"][0], f"prefill slot {b}", **tl)
    teach = synth.prompts(c, B, 2, stream=synth.TEACHER_STREAM)
    for s in range(2):
        hid, _, _ = pair.capture_buffers(B)
        lg = pair.gpu.decode(teach[:, s].tolist(), [P + s] * B).cpu().numpy()
        r = pair.ora.decode(teach[:, s].tolist(), [P + s] * B, capture=True)
        torch.cuda.synchronize()
        h = hid.cpu().numpy()
        for b in range(B):
            rl = rel_l2(h[1, b], r["hidden"][1, b])
            assert rl <= HIDDEN_REL_L2, f"decode step {s} row {b}: hidden rel L2 {rl:.3e}"
            check_logits(lg[b], r["logits"][b], f"decode step {s} row {b}", **tl)
            check_argmax(lg[b], r["logits"][b], f"decode step {s} row {b}", **tl)


WIDE_Q = configs.ModelConfig("wide-q-1l", n_layers=1, hidden=512, n_heads=32, n_kv_heads=8, head_dim=128,
                             ffn_dim=1024, vocab=1000, max_seq=4096, rms_eps=1e-5, rope_theta=1e4)


def test_gemm_two_way_k_split_with_a_token_tail():
    """q|k|v of 6144 features over 2800 tokens is 24 x 11 = 264 tiles of 256 x 256:
    a second round of 8 tiles, so the projection is split in two over k (528
    blocks) and the RoPE/KV pass sums the two partials; the last token tile
    holds 240 rows."""
    pair = Pair(WIDE_Q, max_prefill=2800, max_seq=4096)
    toks = synth.tokens(0, synth.PROMPT_STREAM, 2800, WIDE_Q.vocab).tolist()
    _chunks(pair, toks, [2800], "two-way k split")


def test_grouped_expert_projections_at_every_row_tile_count():
    """bf16 experts through the grouped LDS-ring GEMV with 1, 3 and 8 column
    tiles of 8 rows: a 40-token prefill (each expert takes up to 40 rows), then
    decode steps at B = 64 (the maximum), 24 and 5; experts, every row's hidden
    state after each layer and the logits against the oracle."""
    cfg = configs.TINY_BF16.replace(name="tiny-bf16-moe-64", n_experts=8, top_k=2, max_seq=64)
    B, P = 64, 40
    pair = Pair(cfg, n_slots=B, max_prefill=P, max_seq=64)
    tl = pair.tol
    hid, ids, rl = pair.capture_buffers(P)
    first = synth.prompts(cfg, 1, P)[0].tolist()
    g = pair.gpu.prefill(first, seq=0).cpu().numpy()
    r = pair.ora.prefill(first, slot=0, capture=True)
    torch.cuda.synchronize()
    check_logits(g, r["logits"][0], "prefill 40", **tl)
    check_experts(ids.cpu().numpy(), r["ids"], r["router"], cfg.top_k, "prefill 40")
    h = hid.cpu().numpy()
    for l in range(cfg.n_layers + 1):
        for t in range(P):
            rl2 = rel_l2(h[l, t], r["hidden"][l, t])
            assert rl2 <= HIDDEN_REL_L2, f"prefill 40: layer {l - 1} row {t} hidden rel L2 {rl2:.3e}"
    pair.gpu.set_capture(None, None, None)
    short = synth.prompts(cfg, B, 3)
    for b in range(1, B):
        pair.gpu.prefill(short[b].tolist(), seq=b)
        pair.ora.prefill(short[b].tolist(), slot=b)
    lens = [P] + [3] * (B - 1)
    teach = synth.prompts(cfg, B, 3, stream=synth.TEACHER_STREAM)
    for s, rows in enumerate((64, 24, 5)):
        hid, ids, rl = pair.capture_buffers(rows)
        toks = teach[:rows, s].tolist()
        pos = lens[:rows]
        lg = pair.gpu.decode(toks, pos).cpu().numpy()
        r = pair.ora.decode(toks, pos, capture=True)
        torch.cuda.synchronize()
        what = f"decode B={rows}"
        check_experts(ids.cpu().numpy(), r["ids"], r["router"], cfg.top_k, what)
        check_hidden(hid.cpu().numpy(), r["hidden"], what)
        for b in range(rows):
            check_logits(lg[b], r["logits"][b], f"{what} row {b}", **tl)
        for b in range(rows):
            lens[b] += 1
