"""Parity of the 24-bit K/V cache (kv_dtype = DEC_KV_F24).

Each rotated key and each value is rounded to nearest even at 16 significant
bits when stored (fp32's sign and exponent with 15 stored mantissa bits) and
kept as 3 bytes; every later read rebuilds that fp32 word exactly (rml "The
decoder", section "Attend": the cache's element type is a switch, rows are
widened to fp32 as they are read).  16 significant bits is what the bf16
(hi, lo) pair of an fp32 value carries into the MFMA attention kernels, so
the cache keeps what those products use.  The oracle mirrors the rounding at
store (pinned on the CPU against an independent rounding); the tolerances are
the fp32 cache's (rel L2 1e-3 on logits and hidden states, argmax margin
1e-3), and the last tests hold the GPU to the plain fp32-cache oracle under
the same tolerances.  Covered: the lane-group decode kernel (head_dim 16 and
128, 3:1 and 4:1 groups, the ring wrap), the MFMA decode form (7:1 groups),
the tile-image MFMA prefill (head_dim 64 and 128), the general prefill kernel
and the fp32 scalar prefill kernel (head_dim 16).
"""
import numpy as np
import pytest
import torch

from decoder_only_forward_amd import configs, synth
from decoder_only_forward_amd.dec import DecModel
from oracle import oracle as O
from parity_util import Pair, check_argmax, check_hidden, check_logits, to_device
from test_gpu_fullwidth import _run
from test_gpu_parity import _run_stream

pytestmark = pytest.mark.gpu

TINY_SET = [configs.TINY_KVF24,
            configs.TINY.replace(name="tiny-f32w-kvf24", kv_f24=True),
            configs.TINY_MOE.replace(name="tiny-moe-kvf24", kv_f24=True),
            configs.TINY_HALF.replace(name="tiny-half-kvf24", kv_f24=True),
            configs.TINY_BIAS.replace(name="tiny-bias-kvf24", kv_f24=True)]


@pytest.mark.parametrize("cfg", TINY_SET, ids=lambda c: c.name)
def test_tiny_f24_cache_prefill_then_greedy_decode(cfg):
    pair = Pair(cfg, max_prefill=8)
    prompt = synth.tokens(0, synth.PROMPT_STREAM, 8, cfg.vocab).tolist()
    _run_stream(pair, prompt, 8, cfg.name)


def test_tiny_f24_cache_ring_wrap():
    cfg = configs.TINY_WINDOW.replace(name="tiny-window-kvf24", kv_f24=True)
    prompt = synth.tokens(0, synth.PROMPT_STREAM, 4, cfg.vocab).tolist()
    _run_stream(Pair(cfg, max_prefill=16), prompt, 11, "f24 ring decode")


def test_smollm2_f24_cache_prefill_128_and_decode_b1():
    cfg = configs.SMOLLM2.replace(name="smollm2-kvf24", kv_f24=True)
    pair = Pair(cfg, max_prefill=128)
    prompt = synth.tokens(0, synth.PROMPT_STREAM, 128, cfg.vocab).tolist()
    _run_stream(pair, prompt, 4, cfg.name)


def test_smollm2_f24_cache_decode_b32():
    cfg = configs.SMOLLM2.replace(name="smollm2-kvf24", kv_f24=True)
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
            check_logits(g[b], r["logits"][b], f"row {b} step {s}", **pair.tol)
            check_argmax(g[b], r["logits"][b], f"row {b} step {s}", **pair.tol)
        nxt = [int(np.argmax(r["logits"][b])) for b in range(B)]


def test_mistral_one_layer_f24_cache_decode_b32_at_full_ring():
    """The throughput workload's decode launch on a 24-bit cache: 32 rows after
    4096-token prompts, each reading a full 4096-slot ring."""
    cfg = configs.one_layer(configs.MISTRAL).replace(name="mistral-1l-kvf24", kv_f24=True)
    _run(cfg, P=4096, B=32, steps=2, sample_rows=[0, 64, 4095], decode_rows=[0, 31], sample_steps={0, 1})


def test_mistral_one_layer_f24_cache_decode_b8_and_b1_through_ring_wrap():
    cfg = configs.one_layer(configs.MISTRAL).replace(name="mistral-1l-kvf24", kv_f24=True)
    _run(cfg, P=4096, B=8, steps=6, sample_rows=[2049, 4095], decode_rows=[0, 7], sample_steps={0, 5})
    _run(cfg, P=4096, B=1, steps=3, sample_rows=[4095], decode_rows=[0], sample_steps={0, 2})


def test_qwen25_one_layer_f24_cache_prefill_2048_and_decode_b64_b1():
    """7:1 groups: the MFMA decode form reading 24-bit rows."""
    cfg = configs.one_layer(configs.QWEN25).replace(name="qwen25-1l-kvf24", kv_f24=True)
    _run(cfg, P=2048, B=64, steps=3, sample_rows=[0, 127, 128, 2047], decode_rows=[0, 63], sample_steps={0, 2})
    _run(cfg, P=2048, B=1, steps=3, sample_rows=[2047], decode_rows=[0], sample_steps={0, 2})


def test_f24_cache_differs_from_fp32_cache():
    """The switch is live: the same model with an fp32 cache gives different
    (though close) logits, so the tests above do not pass vacuously."""
    cfg = configs.TINY_KVF24
    prompt = synth.tokens(0, synth.PROMPT_STREAM, 8, cfg.vocab).tolist()
    a = Pair(cfg, max_prefill=8).gpu.prefill(prompt).cpu().numpy()
    b = Pair(cfg.replace(kv_f24=False), max_prefill=8).gpu.prefill(prompt).cpu().numpy()
    assert not np.array_equal(a, b)
    check_logits(a, b, "f24 vs fp32 cache")


@pytest.mark.parametrize("steps,B", [(4, 1), (2, 8)])
def test_smollm2_f24_cache_against_fp32_cache_oracle(steps, B):
    """The 24-bit cache against the plain oracle (fp32 cache, no rounding at
    store) under the fp32 tolerances, every layer's hidden state and logits,
    at full depth: prefill of 128 tokens, then batched decode."""
    cfg = configs.SMOLLM2.replace(name="smollm2-kvf24", kv_f24=True)
    w = synth.make_weights(cfg)
    gpu = DecModel(cfg, to_device(w), max_batch=B, max_prefill=128)
    ora = O.OracleModel(cfg.replace(kv_f24=False), w, n_slots=B, kind="f32")
    pr = synth.prompts(cfg, B, 128)
    nxt = []
    for b in range(B):
        g = gpu.prefill(pr[b].tolist(), seq=b).cpu().numpy()
        r = ora.prefill(pr[b].tolist(), slot=b)
        check_logits(g, r["logits"][0], f"prefill slot {b}")
        nxt.append(int(np.argmax(r["logits"][0])))
    for s in range(steps):
        hid = torch.full((cfg.n_layers + 1, B, cfg.hidden), float("nan"), device="cuda")
        gpu.set_capture(hid, None, None)
        g = gpu.decode(nxt, [128 + s] * B).cpu().numpy()
        r = ora.decode(nxt, [128 + s] * B, capture=True)
        gpu.set_capture(None, None, None)
        h = hid.cpu().numpy()
        for b in range(B):
            check_logits(g[b], r["logits"][b], f"step {s} row {b}")
            check_argmax(g[b], r["logits"][b], f"step {s} row {b}")
            check_hidden(h[:, b], r["hidden"][:, b], f"step {s} row {b}")
        nxt = [int(np.argmax(r["logits"][b])) for b in range(B)]
    gpu.close()
