"""Full-width parity: one-layer models with every kernel at its real size.

Each model keeps the full hidden, head, FFN and vocabulary sizes of its shape
but a single layer, so the CPU oracle can recompute sampled rows on its own
(rows a prefill does not sample still get their K/V, which later rows read).
The GPU runs the workload's launch configuration (prefill of P tokens, then
batched decode through the ring wrap where the shape has a window); the oracle
reproduces sampled decode rows as rows of one prefill over the same token
sequence (single-pass prefill equals per-token forward, sipllm "Transformer
forward pass", section "Single-pass prefill").

Weights are drawn on the GPU (the generator test below pins GPU draws to CPU
draws bit for bit) and copied to the host for the oracle.
"""
import numpy as np
import pytest
import torch

from decoder_only_forward_amd import configs, synth
from decoder_only_forward_amd.dec import DecModel
from oracle import oracle as O
from parity_util import check_argmax, check_experts, check_logits, oracle_kind, rel_l2, tol, HIDDEN_REL_L2

pytestmark = pytest.mark.gpu


def test_generator_gpu_draws_equal_cpu_draws():
    for dt, n, tid in ((torch.bfloat16, 1 << 20, 1234), (torch.float32, 4099, 17)):
        a = torch.empty(n, dtype=dt, device="cuda")
        b = torch.empty(n, dtype=dt)
        synth.fill_normal(a, 0, tid, 0.02, chunk=1 << 18)
        synth.fill_normal(b, 0, tid, 0.02)
        ia = a.cpu().view(torch.int16 if dt == torch.bfloat16 else torch.int32)
        ib = b.view(torch.int16 if dt == torch.bfloat16 else torch.int32)
        assert torch.equal(ia, ib)
    assert torch.equal(synth.tokens(0, 7, 5000, 32000, "cuda").cpu(), synth.tokens(0, 7, 5000, 32000))


def _host(wd):
    w = {k: (v.cpu() if v is not None else None) for k, v in wd.items() if k != "layers"}
    w["layers"] = [{k: v.cpu() for k, v in lw.items()} for lw in wd["layers"]]
    return w


def _run(cfg, P, B, steps, sample_rows, decode_rows, sample_steps):
    """Prefill P prompt tokens into each of B slots (row 0 with hidden capture),
    then `steps` decode steps at batch B with seeded teacher tokens."""
    torch.manual_seed(0)
    wd = synth.make_weights(cfg, seed=0, device="cuda")
    w = _host(wd)
    gpu = DecModel(cfg, wd, max_batch=B, max_prefill=P)
    prompts = synth.prompts(cfg, B, P)
    teach = synth.prompts(cfg, B, steps, stream=synth.TEACHER_STREAM)
    hid = torch.full((2, P, cfg.hidden), float("nan"), device="cuda")
    ids = router = None
    if cfg.n_experts:
        ids = torch.zeros((1, P, cfg.top_k), dtype=torch.int32, device="cuda")
        router = torch.zeros((1, P, cfg.n_experts), device="cuda")
    gpu.set_capture(hid, ids, router)
    pre_logits = gpu.prefill(prompts[0].tolist(), seq=0).cpu().numpy()
    gpu.set_capture(None, None, None)
    for b in range(1, B):
        gpu.prefill(prompts[b].tolist(), seq=b)
    dec_logits = {}
    for s in range(steps):
        lg = gpu.decode(teach[:, s].tolist(), [P + s] * B)
        if s in sample_steps:
            dec_logits[s] = lg.cpu().numpy()
    torch.cuda.synchronize()
    hid = hid.cpu().numpy()

    # oracle: row 0's prefill with sampled rows
    tl = tol(cfg)
    hid_tol = HIDDEN_REL_L2 if not cfg.kv_bf16 else tl["rel"]
    ora = O.OracleModel(cfg, w, n_slots=1, max_seq=cfg.max_seq, kind=oracle_kind(cfg))
    r = ora.prefill(prompts[0].tolist(), rows=sample_rows, partial=True, capture=True)
    for i, t in enumerate(sample_rows):
        rl = rel_l2(hid[1, t], r["hidden"][1, t])
        assert rl <= hid_tol, f"{cfg.name} prefill row {t}: hidden rel L2 {rl:.3e}"
    check_logits(pre_logits, r["logits"][-1], f"{cfg.name} prefill logits", **tl)
    check_argmax(pre_logits, r["logits"][-1], f"{cfg.name} prefill argmax", **tl)
    if cfg.n_experts:
        gi = ids.cpu().numpy()[:, sample_rows]
        check_experts(gi, r["ids"][:, sample_rows], r["router"][:, sample_rows], cfg.top_k, f"{cfg.name} experts")
    # oracle: decode rows as rows of one prefill over prompt + teacher tokens
    for b in decode_rows:
        seq = prompts[b].tolist() + teach[b].tolist()
        rows = [P + s for s in sorted(sample_steps)]
        ob = O.OracleModel(cfg, w, n_slots=1, max_seq=cfg.max_seq, kind=oracle_kind(cfg))
        rb = ob.prefill(seq, rows=rows, partial=True)
        for i, s in enumerate(sorted(sample_steps)):
            check_logits(dec_logits[s][b], rb["logits"][i], f"{cfg.name} decode row {b} step {s}", **tl)
            check_argmax(dec_logits[s][b], rb["logits"][i], f"{cfg.name} decode row {b} step {s}", **tl)
    gpu.close()


def test_qwen25_one_layer_prefill_2048_and_decode_b64():
    """Qwen2.5-0.5B width (7:1 GQA, q/k/v bias, theta 1e6, eps 1e-6, tied head)."""
    cfg = configs.one_layer(configs.QWEN25)
    _run(cfg, P=2048, B=64, steps=4, sample_rows=[0, 1, 127, 128, 1000, 2047],
         decode_rows=[0, 63], sample_steps={0, 3})


def test_mistral_one_layer_prefill_4096_and_decode_through_ring_wrap():
    """Mistral-7B width (head_dim 128, 4:1 GQA), 4096-slot ring: decode from
    position 4096 overwrites slot 0 and reads positions 1..4096."""
    cfg = configs.one_layer(configs.MISTRAL)
    _run(cfg, P=4096, B=8, steps=6, sample_rows=[0, 63, 64, 2049, 4095],
         decode_rows=[0, 7], sample_steps={0, 5})


def test_mixtral_one_layer_prefill_512_and_decode_b16():
    """Mixtral-8x7B width: 8 experts of ffn 14336, top-2; grouped experts read
    only the selected experts."""
    cfg = configs.one_layer(configs.MIXTRAL)
    _run(cfg, P=512, B=16, steps=3, sample_rows=[0, 5, 255, 511],
         decode_rows=[0, 15], sample_steps={0, 2})


def test_mistral_one_layer_llama3_scaling_and_half_pairing():
    """RoPE variants at head_dim 128: llama3 frequency scaling (factor 8,
    low/high 1/4, original context 8192) with rotate-half pairing."""
    cfg = configs.one_layer(configs.MISTRAL).replace(name="mistral-1l-llama3-half", rope_pairing=1,
                                                      rope_scaling=1, rope_orig_ctx=8192, rope_factor=8.0)
    _run(cfg, P=1024, B=2, steps=3, sample_rows=[0, 511, 1023], decode_rows=[1], sample_steps={0, 2})


def test_qwen25_one_layer_decode_b1_after_2048():
    """Qwen2.5-0.5B width at the workload's batch 1: decode at positions
    2048.. reads 2049+ keys of one kv head for seven query heads, the new key's
    slot inside one of the attention splits."""
    cfg = configs.one_layer(configs.QWEN25)
    _run(cfg, P=2048, B=1, steps=4, sample_rows=[2047], decode_rows=[0], sample_steps={0, 1, 3})


def test_mixtral_one_layer_decode_b1_after_512():
    """Mixtral-8x7B width at the workload's batch 1: each step's two experts
    hold one row each in the grouped expert GEMV (K = 4096 and 14336)."""
    cfg = configs.one_layer(configs.MIXTRAL)
    _run(cfg, P=512, B=1, steps=3, sample_rows=[511], decode_rows=[0], sample_steps={0, 1, 2})


def test_mistral_one_layer_decode_b32_at_full_ring():
    """The Mistral-7B decode launch of the throughput workload: 32 rows, each
    after a 4096-token prompt, so every row reads a full 4096-slot ring (one
    attention split per row and kv head) and overwrites slot 0, then 1."""
    cfg = configs.one_layer(configs.MISTRAL)
    _run(cfg, P=4096, B=32, steps=2, sample_rows=[4095], decode_rows=[0, 31], sample_steps={0, 1})


def test_mistral_one_layer_decode_b1_at_full_ring():
    """Mistral-7B width at batch 1 after a 4096-token prompt: the attention
    runs in 32 splits per kv head and the output projection's blocks merge
    them (one split range holds the overwritten ring slot)."""
    cfg = configs.one_layer(configs.MISTRAL)
    _run(cfg, P=4096, B=1, steps=3, sample_rows=[4095], decode_rows=[0], sample_steps={0, 1, 2})
