"""Parity of the prefill projections on fp16 + fp8 split operands
(DEC_PREFILL_F16_F8) against the oracle, at the tolerance of the fp32 path.

In that form a prefill of more than 64 rows runs each q|k|v projection, and
each fused gate|up projection large enough for the direct-to-LDS kernel, as
an fp16 pass against an fp16 copy of the weights plus a scaled fp8 pass
against an fp8 copy.  The residual + RMSNorm before them writes that operand
form; the other projections (o, down, the LM head, MoE experts) keep the bf16
pair.  The oracle computes the forward itself (Pantheon "Llama Forward Pass",
section "Forward Pass Flow"), unaware of the operand form, so these runs hold
the form to the same bound as the bf16 pair.

- Mistral-7B, Qwen2.5-0.5B and Mixtral-8x7B widths at one layer and the
  workloads' prompt lengths, then decode steps reading the K/V the prefill
  wrote (the full-width harness of test_gpu_fullwidth.py).
- Qwen2.5-0.5B width at two layers: the form passes from layer to layer
  (the second layer's norm writes it for the second q|k|v) and the last norm
  hands the LM head the bf16 pair; every row's hidden state and logits.
- A SmolLM2-135M-width model at full depth with 128-token prompts: q|k|v in
  the form, the FFN too small for the fused kernel (bf16 pair).
"""
import numpy as np
import pytest

from decoder_only_forward_amd import configs, synth
from parity_util import Pair, check_argmax, check_hidden, check_logits
from test_gpu_fullwidth import _run

pytestmark = pytest.mark.gpu


def _f8(cfg, name):
    return cfg.replace(name=name, prefill_fp8=True)


def test_mistral_one_layer_prefill_4096_f8():
    print("[prefill f8] mistral-7b 1 layer P=4096", flush=True)
    cfg = _f8(configs.one_layer(configs.MISTRAL), "mistral-7b-1l-f8")
    _run(cfg, P=4096, B=2, steps=2, sample_rows=[0, 63, 64, 255, 256, 2049, 4095], decode_rows=[1],
         sample_steps={0, 1})


def test_qwen25_one_layer_prefill_2048_f8():
    print("[prefill f8] qwen2.5-0.5b 1 layer P=2048", flush=True)
    cfg = _f8(configs.one_layer(configs.QWEN25), "qwen2.5-0.5b-1l-f8")
    _run(cfg, P=2048, B=2, steps=2, sample_rows=[0, 1, 127, 128, 1000, 2047], decode_rows=[0],
         sample_steps={0, 1})


def test_mixtral_one_layer_prefill_512_f8():
    print("[prefill f8] mixtral-8x7b 1 layer P=512", flush=True)
    cfg = _f8(configs.one_layer(configs.MIXTRAL), "mixtral-8x7b-1l-f8")
    _run(cfg, P=512, B=2, steps=2, sample_rows=[0, 5, 255, 511], decode_rows=[1], sample_steps={0, 1})


@pytest.mark.parametrize("P", [2048, 1000])
def test_qwen25_two_layers_every_row_f8(P):
    """P = 2048: 304 fused gate|up tiles (the form); P = 1000: 152 tiles, so
    the FFN keeps the bf16 pair while q|k|v take the form, with a ragged last
    256-row tile."""
    cfg = _f8(configs.QWEN25.replace(n_layers=2, vocab=512, tied_embedding=False), f"qwen-2l-f8-p{P}")
    print(f"[prefill f8] {cfg.name}", flush=True)
    pair = Pair(cfg, max_prefill=P, max_seq=P + 8)
    toks = synth.tokens(0, synth.PROMPT_STREAM, P, cfg.vocab).tolist()
    hid, _, _ = pair.capture_buffers(P)
    g = pair.gpu.prefill(toks, start_pos=0, all_logits=True).cpu().numpy()
    r = pair.ora.prefill(toks, start_pos=0, rows=list(range(P)), capture=True)
    for t in range(0, P, 97):
        check_logits(g[t], r["logits"][t], f"{cfg.name} row {t}", **pair.tol)
        check_argmax(g[t], r["logits"][t], f"{cfg.name} row {t}", **pair.tol)
    check_logits(g[P - 1], r["logits"][P - 1], f"{cfg.name} row {P - 1}", **pair.tol)
    check_hidden(hid.cpu().numpy(), r["hidden"], cfg.name, **pair.tol)
    nxt = int(np.argmax(r["logits"][-1]))
    gd = pair.gpu.decode([nxt], [P]).cpu().numpy()[0]
    rd = pair.ora.decode([nxt], [P])["logits"][0]
    check_logits(gd, rd, f"{cfg.name} decode after the prefill", **pair.tol)


def test_smollm2_full_depth_prefill_128_f8():
    cfg = _f8(configs.SMOLLM2.replace(max_seq=256), "smollm2-f8")
    print(f"[prefill f8] {cfg.name} full depth P=128", flush=True)
    P = 128
    pair = Pair(cfg, max_prefill=P, max_seq=256)
    toks = synth.tokens(0, synth.PROMPT_STREAM, P, cfg.vocab).tolist()
    hid, _, _ = pair.capture_buffers(P)
    g = pair.gpu.prefill(toks, start_pos=0).cpu().numpy()
    rows = [0, 64, 127]
    r = pair.ora.prefill(toks, start_pos=0, rows=rows, capture=True)
    check_logits(g, r["logits"][-1], f"{cfg.name} last row", **pair.tol)
    check_argmax(g, r["logits"][-1], f"{cfg.name} last row", **pair.tol)
    check_hidden(hid.cpu().numpy()[:, rows], r["hidden"][:, rows], cfg.name, **pair.tol)
