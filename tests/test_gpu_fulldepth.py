"""Full-depth parity for the three largest shapes: every layer at full width,
the workload's decode batch, and a short prompt.

The CPU oracle streams the bf16 weights once per token, so a full-depth row
costs it about a second for Mixtral-8x7B (two experts a layer) and a quarter
second for Mistral-7B; the workloads' full prompt lengths (2048 / 4096 / 512)
are covered at full width by the one-layer tests instead.

Per model: prefill P prompt tokens into each of B sequence slots (row 0 with
every layer's hidden state and, for the MoE shape, the selected experts
captured), then `steps` decode steps at batch B with teacher-forced tokens.
The oracle replays row 0: the same prefill, compared on the hidden state of
sampled positions after every layer, the expert ids of every position and
layer, and the last position's logits and greedy token; then the same decode
steps one token at a time, compared on logits, greedy token and every layer's
hidden state of row 0.
"""
import numpy as np
import pytest
import torch

from decoder_only_forward_amd import configs, synth
from decoder_only_forward_amd.dec import DecModel
from oracle import oracle as O
from parity_util import HIDDEN_REL_L2, check_argmax, check_experts, check_logits, rel_l2, tol

pytestmark = pytest.mark.gpu


def _run(cfg, P, B, steps, rows):
    c = cfg
    wd = synth.make_weights(cfg, seed=0, device="cuda")
    gpu = DecModel(cfg, wd, max_batch=B, max_prefill=P)
    prompts = synth.prompts(cfg, B, P)
    teach = synth.prompts(cfg, B, steps, stream=synth.TEACHER_STREAM)

    hid = torch.full((c.n_layers + 1, P, c.hidden), float("nan"), device="cuda")
    ids = router = None
    if c.n_experts:
        ids = torch.zeros((c.n_layers, P, c.top_k), dtype=torch.int32, device="cuda")
        router = torch.zeros((c.n_layers, P, c.n_experts), device="cuda")
    gpu.set_capture(hid, ids, router)
    pre = gpu.prefill(prompts[0].tolist(), seq=0).cpu().numpy()
    gpu.set_capture(None, None, None)
    for b in range(1, B):
        gpu.prefill(prompts[b].tolist(), seq=b)
    dec_logits, dec_hid, dec_ids = [], [], []
    for s in range(steps):
        h = torch.full((c.n_layers + 1, B, c.hidden), float("nan"), device="cuda")
        di = torch.zeros((c.n_layers, B, c.top_k), dtype=torch.int32, device="cuda") if c.n_experts else None
        dr = torch.zeros((c.n_layers, B, c.n_experts), device="cuda") if c.n_experts else None
        gpu.set_capture(h, di, dr)
        lg = gpu.decode(teach[:, s].tolist(), [P + s] * B)
        gpu.set_capture(None, None, None)
        dec_logits.append(lg[0].cpu().numpy())
        dec_hid.append(h[:, 0].cpu().numpy())
        dec_ids.append(di[:, 0:1].cpu().numpy() if c.n_experts else None)
    torch.cuda.synchronize()
    hid = hid.cpu().numpy()
    ids = ids.cpu().numpy() if c.n_experts else None
    gpu.close()
    # host copy of the same weights for the oracle; free the device copy
    w = {k: (v.cpu() if v is not None else None) for k, v in wd.items() if k != "layers"}
    w["layers"] = [{k: v.cpu() for k, v in lw.items()} for lw in wd["layers"]]
    del wd, gpu
    torch.cuda.empty_cache()

    tl = tol(cfg)
    ora = O.OracleModel(cfg, w, n_slots=1, max_seq=cfg.max_seq)
    r = ora.prefill(prompts[0].tolist(), capture=True)
    for t in rows:
        for l in range(c.n_layers + 1):
            rl = rel_l2(hid[l, t], r["hidden"][l, t])
            assert rl <= HIDDEN_REL_L2, f"{c.name} prefill row {t}: hidden after layer {l - 1} rel L2 {rl:.3e}"
    check_logits(pre, r["logits"][0], f"{c.name} prefill logits", **tl)
    check_argmax(pre, r["logits"][0], f"{c.name} prefill argmax", **tl)
    if c.n_experts:
        check_experts(ids, r["ids"], r["router"], c.top_k, f"{c.name} prefill experts")
    for s in range(steps):
        rd = ora.decode([int(teach[0, s])], [P + s], capture=True)
        what = f"{c.name} decode row 0 step {s}"
        check_logits(dec_logits[s], rd["logits"][0], what, **tl)
        check_argmax(dec_logits[s], rd["logits"][0], what, **tl)
        for l in range(c.n_layers + 1):
            rl = rel_l2(dec_hid[s][l], rd["hidden"][l, 0])
            assert rl <= HIDDEN_REL_L2, f"{what}: hidden after layer {l - 1} rel L2 {rl:.3e}"
        if c.n_experts:
            check_experts(dec_ids[s], rd["ids"], rd["router"], c.top_k, what)


def test_qwen25_full_depth_prefill_512_and_decode_b64():
    """Qwen2.5-0.5B: 24 layers, 7:1 GQA, q/k/v biases, theta 1e6, tied head."""
    _run(configs.QWEN25, P=512, B=64, steps=3, rows=[0, 255, 511])


def test_mistral_full_depth_prefill_64_and_decode_b32():
    """Mistral-7B: 32 layers, head_dim 128, 4096-slot ring cache."""
    _run(configs.MISTRAL, P=64, B=32, steps=2, rows=[0, 63])


def test_mixtral_full_depth_prefill_32_and_decode_b16():
    """Mixtral-8x7B: 32 layers of 8 experts (top-2), ~93 GB of bf16 weights."""
    _run(configs.MIXTRAL, P=32, B=16, steps=2, rows=[0, 31])
