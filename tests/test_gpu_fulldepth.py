"""Full-depth parity for the three largest shapes: every layer at full width,
the workload's decode batch, and a short prompt.

The CPU oracle streams the bf16 weights once per token, so a full-depth row
costs it about a second for Mixtral-8x7B (two experts a layer) and a quarter
second for Mistral-7B; the workloads' full prompt lengths (2048 / 4096 / 512)
are covered at full width by the one-layer tests instead.

Per model: prefill P prompt tokens into each of B sequence slots (row 0 with
every layer's hidden state and, for the MoE shape, the selected experts
captured), then `steps` decode steps at batch B with teacher-forced tokens.
The same rows then run one at a time on a second handle with one slot (decode
at B = 1, the workloads' other batch size): every row's logits at every step
must agree with the batched run.  The oracle replays sampled rows (row 0, the
middle and the last row): the same prefill, compared for row 0 on the hidden
state of sampled positions after every layer, the expert ids of every position
and layer, and the last position's logits and greedy token; then the same
decode steps one token at a time, compared on logits, greedy token, every
layer's hidden state and (MoE) expert ids of the batched run and of the B = 1
run.  (Pantheon "Llama Forward Pass", section "Batched Multi-Sequence Decode":
rows are independent sequences.)
"""
import numpy as np
import pytest
import torch

from decoder_only_forward_amd import configs, synth
from decoder_only_forward_amd.dec import DecModel
from oracle import oracle as O
from parity_util import HIDDEN_REL_L2, check_argmax, check_experts, check_logits, rel_l2, tol

pytestmark = pytest.mark.gpu


def _decode_capture(gpu, c, B, toks, pos):
    h = torch.full((c.n_layers + 1, B, c.hidden), float("nan"), device="cuda")
    di = torch.zeros((c.n_layers, B, c.top_k), dtype=torch.int32, device="cuda") if c.n_experts else None
    dr = torch.zeros((c.n_layers, B, c.n_experts), device="cuda") if c.n_experts else None
    gpu.set_capture(h, di, dr)
    lg = gpu.decode(toks, pos)
    gpu.set_capture(None, None, None)
    torch.cuda.synchronize()
    return (lg.cpu().numpy(), h.cpu().numpy(), di.cpu().numpy() if c.n_experts else None)


def _run(cfg, P, B, steps, rows, oracle_rows):
    c = cfg
    tl = tol(cfg)
    print(f"[fulldepth] {c.name} P={P} B={B} steps={steps}", flush=True)
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
    batched = [_decode_capture(gpu, c, B, teach[:, s].tolist(), [P + s] * B) for s in range(steps)]
    hid = hid.cpu().numpy()
    ids = ids.cpu().numpy() if c.n_experts else None
    gpu.close()
    del gpu

    # the same rows one at a time (decode at B = 1)
    one = DecModel(cfg, wd, max_batch=1, max_prefill=P)
    single = {}
    for b in range(B):
        one.reset()
        one.prefill(prompts[b].tolist(), seq=0)
        outs = [_decode_capture(one, c, 1, [int(teach[b, s])], [P + s]) for s in range(steps)]
        for s in range(steps):
            what = f"{c.name} row {b} step {s}: B = 1 vs batched"
            check_logits(outs[s][0][0], batched[s][0][b], what, **tl)
            check_argmax(outs[s][0][0], batched[s][0][b], what, **tl)
        if b in oracle_rows:
            single[b] = outs
    one.close()
    del one
    # host copy of the same weights for the oracle; free the device copy
    w = {k: (v.cpu() if v is not None else None) for k, v in wd.items() if k != "layers"}
    w["layers"] = [{k: v.cpu() for k, v in lw.items()} for lw in wd["layers"]]
    del wd
    torch.cuda.empty_cache()

    for b in oracle_rows:
        ora = O.OracleModel(cfg, w, n_slots=1, max_seq=cfg.max_seq)
        r = ora.prefill(prompts[b].tolist(), capture=(b == 0))
        if b == 0:
            for t in rows:
                for l in range(c.n_layers + 1):
                    rl = rel_l2(hid[l, t], r["hidden"][l, t])
                    assert rl <= HIDDEN_REL_L2, f"{c.name} prefill row {t}: hidden after layer {l - 1} rel L2 {rl:.3e}"
            check_logits(pre, r["logits"][0], f"{c.name} prefill logits", **tl)
            check_argmax(pre, r["logits"][0], f"{c.name} prefill argmax", **tl)
            if c.n_experts:
                check_experts(ids, r["ids"], r["router"], c.top_k, f"{c.name} prefill experts")
        for s in range(steps):
            rd = ora.decode([int(teach[b, s])], [P + s], capture=True)
            for name, (lg, h, di), row in (("batched", batched[s], b), ("B = 1", single[b][s], 0)):
                what = f"{c.name} decode row {b} step {s} ({name})"
                check_logits(lg[row], rd["logits"][0], what, **tl)
                check_argmax(lg[row], rd["logits"][0], what, **tl)
                for l in range(c.n_layers + 1):
                    rl = rel_l2(h[l, row], rd["hidden"][l, 0])
                    assert rl <= HIDDEN_REL_L2, f"{what}: hidden after layer {l - 1} rel L2 {rl:.3e}"
                if c.n_experts:
                    check_experts(di[:, row:row + 1], rd["ids"], rd["router"], c.top_k, what)


def test_qwen25_full_depth_prefill_512_and_decode_b64_and_b1():
    """Qwen2.5-0.5B: 24 layers, 7:1 GQA, q/k/v biases, theta 1e6, tied head."""
    _run(configs.QWEN25, P=512, B=64, steps=3, rows=[0, 255, 511], oracle_rows=[0, 32, 63])


def test_mistral_full_depth_prefill_64_and_decode_b32_and_b1():
    """Mistral-7B: 32 layers, head_dim 128, 4096-slot ring cache."""
    _run(configs.MISTRAL, P=64, B=32, steps=2, rows=[0, 63], oracle_rows=[0, 31])


def test_mixtral_full_depth_prefill_32_and_decode_b16_and_b1():
    """Mixtral-8x7B: 32 layers of 8 experts (top-2), ~93 GB of bf16 weights."""
    _run(configs.MIXTRAL, P=32, B=16, steps=2, rows=[0, 31], oracle_rows=[0, 15])
