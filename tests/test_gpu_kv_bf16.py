"""Parity of the bf16 K/V cache with the oracle's bf16 mirror.

With kv_dtype = bf16 every rotated key and every value is rounded to the
nearest-even bf16 when stored, and every later read sees the rounded value
(rml "The decoder", section "Attend": the cache's element type is a switch and
rows are widened to fp32 as they are read).  The oracle applies the same
rounding at the same point; the GPU is compared with its fp64 instantiation
under the bf16-cache bound (4u = 2^-7 on logits and hidden states, u the bf16
unit roundoff; see parity_util).  The rounding itself is pinned on the CPU
against torch's nearest-even conversion.  Covered: the fp32 attention kernels (head_dim 16),
the bf16-operand MFMA prefill and the bf16 split-KV decode at head_dim 64
(3:1 and 7:1 groups) and 128 (4:1, through the ring wrap).
"""
import numpy as np
import pytest
import torch

from decoder_only_forward_amd import configs, synth
from parity_util import KV_BF16_REL_L2, Pair, check_argmax, check_logits
from test_gpu_fullwidth import _run
from test_gpu_parity import _run_stream

pytestmark = pytest.mark.gpu

TINY_SET = [configs.TINY_KVBF16,
            configs.TINY.replace(name="tiny-f32w-kvbf16", kv_bf16=True),
            configs.TINY_MOE.replace(name="tiny-moe-kvbf16", kv_bf16=True),
            configs.TINY_HALF.replace(name="tiny-half-kvbf16", kv_bf16=True)]


@pytest.mark.parametrize("cfg", TINY_SET, ids=lambda c: c.name)
def test_tiny_bf16_cache_prefill_then_greedy_decode(cfg):
    pair = Pair(cfg, max_prefill=8)
    prompt = synth.tokens(0, synth.PROMPT_STREAM, 8, cfg.vocab).tolist()
    _run_stream(pair, prompt, 8, cfg.name)


def test_tiny_bf16_cache_ring_wrap():
    cfg = configs.TINY_WINDOW.replace(name="tiny-window-kvbf16", kv_bf16=True)
    prompt = synth.tokens(0, synth.PROMPT_STREAM, 4, cfg.vocab).tolist()
    _run_stream(Pair(cfg, max_prefill=16), prompt, 11, "bf16 ring decode")


def test_smollm2_bf16_cache_prefill_128_and_decode_b1():
    cfg = configs.SMOLLM2.replace(name="smollm2-kvbf16", kv_bf16=True)
    pair = Pair(cfg, max_prefill=128)
    prompt = synth.tokens(0, synth.PROMPT_STREAM, 128, cfg.vocab).tolist()
    _run_stream(pair, prompt, 4, cfg.name)


def test_smollm2_bf16_cache_decode_b32():
    cfg = configs.SMOLLM2.replace(name="smollm2-kvbf16", kv_bf16=True)
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


def test_mistral_one_layer_bf16_cache_prefill_4096_and_decode_through_ring_wrap():
    cfg = configs.one_layer(configs.MISTRAL).replace(name="mistral-1l-kvbf16", kv_bf16=True)
    _run(cfg, P=4096, B=8, steps=6, sample_rows=[0, 63, 64, 2049, 4095],
         decode_rows=[0, 7], sample_steps={0, 5})


def test_mistral_one_layer_bf16_cache_decode_b1_at_full_ring():
    """Batch 1 on the bf16 cache after 4096 prompt tokens: the MFMA decode
    attention in 64 splits per kv head, merged by the split merge kernel."""
    cfg = configs.one_layer(configs.MISTRAL).replace(name="mistral-1l-kvbf16", kv_bf16=True)
    _run(cfg, P=4096, B=1, steps=3, sample_rows=[4095], decode_rows=[0], sample_steps={0, 1, 2})


def test_qwen25_one_layer_bf16_cache_prefill_1024_and_decode_b16():
    cfg = configs.one_layer(configs.QWEN25).replace(name="qwen25-1l-kvbf16", kv_bf16=True)
    _run(cfg, P=1024, B=16, steps=3, sample_rows=[0, 127, 128, 1023],
         decode_rows=[0, 15], sample_steps={0, 2})


def test_bf16_cache_differs_from_fp32_cache():
    """The switch is live: the same model with an fp32 cache gives different
    (though close) logits, so the bf16 tests above do not pass vacuously."""
    cfg = configs.TINY_KVBF16
    prompt = synth.tokens(0, synth.PROMPT_STREAM, 8, cfg.vocab).tolist()
    a = Pair(cfg, max_prefill=8).gpu.prefill(prompt).cpu().numpy()
    b = Pair(cfg.replace(kv_bf16=False), max_prefill=8).gpu.prefill(prompt).cpu().numpy()
    assert not np.array_equal(a, b)
    check_logits(a, b, "bf16 vs fp32 cache", rel=KV_BF16_REL_L2)
