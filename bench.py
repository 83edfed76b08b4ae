"""Decode and prefill throughput of the decoder forward on one MI355X.

Workload (default): the Mistral-7B shape (32 layers, d 4096, 32/8 heads of 128,
ffn 14336, vocab 32000, 4096-slot ring KV cache), bf16 random-init weights from
the seeded generator, drawn on the GPU.  Setup prefills a 4096-token random
prompt into each of the 32 sequence slots (each call is one prefill sample);
then decode runs at batch 32 at positions 4096.. (past the ring's first wrap).

A step is one batched decode call over all layers (embedding to logits) plus
the greedy choice of the B next tokens (the one device->host copy per step).
`value` = B * K / (time of K steps), the steps replaying a captured HIP graph.
Prefill tok/s = 4096 / (median prefill call).  The roofline objects come from
a second timed region of K steps in which every GEMV and attention launch is
bracketed by HIP events on the library's stream (those steps launch eagerly).

The other shapes' workloads follow in `workloads` (same method, each on its
own seeded weights): SmolLM2-135M (prefill 128, decode B = 32 and 1 from
position 128), Qwen2.5-0.5B (prefill 2048, decode B = 64 and 1 from 2048) and
Mixtral-8x7B (prefill 512, decode B = 16 and 1 from 512).  Each decode carries
the step's HBM roofline (algorithmic bytes of one step over its time: every
weight read once, for MoE the experts the step's tokens chose, the readable
K/V of every row, the K/V rows written, the logits) and its kernels' rooflines.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
    python bench.py --only qwen2.5-0.5b [--phase prefill|decode]   (one workload, for profiling)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# HBM bytes per launch of the measured kernels, from two rocprofv3 --pmc passes
# (FETCH_SIZE, WRITE_SIZE) scaled by what the same counters read for a 1 GiB
# device copy (x2.000 and x1.000): reported only while the kernel's sources hash
# to the ones profiled, and only for the profiled workload.  GEMV and GEMM
# figures are the mean over the launches of one step's mix of projections.
_COMMON = {"decoder_only_forward_amd/csrc/common.h":
           "a08d4f553fd07b7970e5b481899ba0e771341cb515b05933bd0498a71b7869c7"}
_ATTN_SOURCES = dict(_COMMON, **{"decoder_only_forward_amd/csrc/k_attn_decode.hip":
                                 "0f2fd612465bb7cbb947ee0ad3a5ffe3f28fc1e9d7af5722580cdc48688cebfd",
                                 "decoder_only_forward_amd/csrc/kvcache.h":
                                 "b917a66e4ecfcb8f83f86f04cd3aed72acacdc8f768e657cc443a9cc9aa212b4"})
_GEMV_SOURCES = dict(_COMMON, **{"decoder_only_forward_amd/csrc/k_gemv.hip":
                                 "1a0a2991d209dd4af919067425a54230bea3a10e27f96688d06e0025b86b6ee5"})
_GEMM_SOURCES = dict(_COMMON, **{"decoder_only_forward_amd/csrc/k_gemm.hip":
                                 "35831c13a16babcb3c1ade248842e44497a91aad2bb89f9ccf4e9ddf241b8c66"})
_TILES_SOURCES = dict(_COMMON, **{"decoder_only_forward_amd/csrc/k_attn_prefill_tiles.hip":
                                  "27be5b4fc493def0a3d08cbf2e9adc0dfb8cf0482bfed8deadcb94b669819d12",
                                  "decoder_only_forward_amd/csrc/kvcache.h":
                                  "b917a66e4ecfcb8f83f86f04cd3aed72acacdc8f768e657cc443a9cc9aa212b4"})
MEASURED_TRAFFIC = {
    # B = 32 launches: the lane-group kernel (fp32 cache; the 24-bit cache in
    # 8-wave blocks), the MFMA kernel in 8-wave blocks (bf16 cache)
    ("attn_decode_kernel", "fp32"): {"sources": _ATTN_SOURCES, "workload": ("mistral-7b", 32, 4096),
                                     "bytes_per_launch": 1078970933},
    ("attn_decode_mfma_kernel", "bf16"): {"sources": _ATTN_SOURCES, "workload": ("mistral-7b", 32, 4096),
                                          "bytes_per_launch": 541889690},
    ("attn_decode_kernel", "f24"): {"sources": _ATTN_SOURCES, "workload": ("mistral-7b", 32, 4096),
                                    "bytes_per_launch": 810591101},
    ("gemv_decode", "fp32"): {"sources": _GEMV_SOURCES, "workload": ("mistral-7b", 32, 4096),
                              "bytes_per_launch": 121781241},
    ("gemv_decode", "bf16"): {"sources": _GEMV_SOURCES, "workload": ("mistral-7b", 32, 4096),
                              "bytes_per_launch": 121781241},
    ("gemv_decode", "f24"): {"sources": _GEMV_SOURCES, "workload": ("mistral-7b", 32, 4096),
                             "bytes_per_launch": 121781241},
    ("gemm_prefill", "fp32"): {"sources": _GEMM_SOURCES, "workload": ("mistral-7b", 32, 4096),
                               "bytes_per_launch": 1716674994},
    ("attn_prefill", "fp32"): {"sources": _TILES_SOURCES, "workload": ("mistral-7b", 32, 4096),
                               "bytes_per_launch": 267578635},
}
# MFMA counters of the prefill kernels (rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES
# GRBM_GUI_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_BUSY_CYCLES): busy = MFMA-busy
# SIMD cycles over all SIMD cycles of the launch (GRBM_GUI_ACTIVE / 8 XCDs x
# 1024 SIMDs); executed = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 flops per launch
# time, against 2.5 PFLOP/s; clock = GRBM_GUI_ACTIVE / 8 per launch time.  The
# projections are the time-weighted mean over one prefill's mix (q+k+v, o,
# gate|up, down); reported only while the sources hash to the profiled ones.
MEASURED_MFMA = {
    ("gemm_prefill", "fp32"): {"sources": _GEMM_SOURCES, "workload": ("mistral-7b", 32, 4096),
                               "busy": 0.569, "executed_frac": 0.466, "clock_ghz": 1.95},
    ("attn_prefill", "fp32"): {"sources": _TILES_SOURCES, "workload": ("mistral-7b", 32, 4096),
                               "busy": 0.461, "executed_frac": 0.394, "clock_ghz": 2.04},
    # the fp16 + fp8 form (q|k|v and gate|up; o and down on the bf16 pair):
    # executed counts each product's fp16 and fp8 flops (the fp8 pass runs at
    # twice the bf16 rate), against 2.5 PFLOP/s
    ("gemm_prefill_f16f8", "fp32"): {"sources": _GEMM_SOURCES, "workload": ("mistral-7b", 32, 4096),
                                     "busy": 0.491, "executed_frac": 0.506, "clock_ghz": 2.05},
}
BF16_PEAK_TFLOPS = 2500.0
# The other shapes' workloads: (decode batches, prompt length).
OTHER = {"smollm2-135m": ((32, 1), 128), "qwen2.5-0.5b": ((64, 1), 2048), "mixtral-8x7b": ((16, 1), 512)}
METRIC = "decode tok/s + prefill tok/s (Mistral-7B shape) and % of HBM / MFMA roofline"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _measured(table, kernel, workload):
    """The table's entry for kernel (name, cache type) on workload (config name,
    batch, prompt), while the kernel's sources hash to the profiled ones."""
    import hashlib
    m = table.get(kernel)
    if not m or m["workload"] != workload:
        return None
    for rel, sha in m["sources"].items():
        with open(os.path.join(ROOT, rel), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != sha:
                return None
    return m


def measured_traffic(kernel, workload):
    m = _measured(MEASURED_TRAFFIC, kernel, workload)
    return None if m is None else m["bytes_per_launch"]


def measured_mfma(kernel, workload):
    m = _measured(MEASURED_MFMA, kernel, workload)
    if m is None:
        return None
    return {"busy": m["busy"], "executed_frac": m["executed_frac"], "clock_ghz": m["clock_ghz"],
            "source": "rocprofv3 PMC: SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE, SQ_INSTS_VALU_MFMA_MOPS_BF16"}


def cpu_baseline(cfg, wd, B=32, prefill_tokens=32):
    """The oracle, untuned, on the host cores, on the same model (weights copied
    to the host): one batched decode step of B rows (each row its first token,
    so the rows read no cached context), then a prefill of the first
    `prefill_tokens` tokens of the workload's prompt.  The oracle forwards one
    row at a time, streaming every weight per row, so its rate hardly depends
    on B; the 4096 cached positions the GPU's decode rows read would add about
    8 % to its per-row work (attention 2 x 32 heads x 128 x 4096 products per
    layer against 218 M weight products), which this bounded sample leaves out."""
    import numpy as np
    from decoder_only_forward_amd import synth
    from oracle import oracle as O
    O.build(force=False)
    w = {k: (v.cpu() if v is not None else None) for k, v in wd.items() if k != "layers"}
    w["layers"] = [{k: v.cpu() for k, v in lw.items()} for lw in wd["layers"]]
    ora = O.OracleModel(cfg, w, n_slots=B, max_seq=cfg.max_seq)
    toks = synth.prompts(cfg, B, 1)[:, 0].tolist()
    t0 = time.perf_counter()
    ora.decode(toks, [0] * B)
    dt_dec = time.perf_counter() - t0
    ora.reset()
    prompt = synth.prompts(cfg, 1, prefill_tokens)[0].tolist()
    t0 = time.perf_counter()
    ora.prefill(prompt)
    dt_pre = time.perf_counter() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(B / dt_dec, 3), "unit": "tok/s", "cores": threads, "kind": "oracle",
            "prefill_tok_s": round(prefill_tokens / dt_pre, 3),
            "sample": f"{cfg.name} full depth: one decode step at B={B} from an empty cache ({dt_dec:.1f} s), "
                      f"and a prefill of the prompt's first {prefill_tokens} tokens ({dt_pre:.1f} s)"}


def ceilings():
    """Measured ceilings beside the published peaks (libdec_probe.so): a
    streaming read of 4 GiB with non-temporal 16-byte loads, a 1 GiB
    device-to-device copy (read + write bytes), and back-to-back bf16 MFMAs
    (32x32x16, four chains a wave, no loads); mean of 5 timed launches each."""
    import torch
    from decoder_only_forward_amd import probe
    buf = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    ms_r = probe.stream_read(buf, reps=5)
    read = buf.numel() / (ms_r * 1e-3) / 1e9
    del buf
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    ms_c = probe.copy(src, dst, reps=5)
    copy = 2 * src.numel() / (ms_c * 1e-3) / 1e9
    del src, dst
    ms_m, fl = probe.mfma_bf16(iters=4096, reps=5)
    torch.cuda.empty_cache()
    return {"hbm_read_GBps": round(read, 1), "hbm_copy_GBps": round(copy, 1),
            "mfma_bf16_TFLOPs": round(fl / (ms_m * 1e-3) / 1e12, 1),
            "source": "probe kernels of libdec_probe.so (include/dec_probe.h), HIP events"}


def kv_bytes(cfg):
    """Bytes of one cached K or V element: fp32 4, bf16 2, the 24-bit format 3."""
    return 2 if cfg.kv_bf16 else (3 if getattr(cfg, "kv_f24", False) else 4)


def kv_name(cfg):
    return "bf16" if cfg.kv_bf16 else ("f24" if getattr(cfg, "kv_f24", False) else "fp32")


def decode_step_bytes(cfg, B, readable, experts_per_layer=None):
    """Algorithmic HBM bytes of one decode step of B rows: every weight read once
    (for MoE the router and the experts in use: `experts_per_layer`, default
    min(E, B*k)), `readable` cached K/V positions summed over the rows, one K
    and one V row written per row and layer, the logits written."""
    d, q, kv, f, V, L = cfg.hidden, cfg.q_dim, cfg.kv_dim, cfg.ffn_dim, cfg.vocab, cfg.n_layers
    wb = 4 if cfg.weight_dtype == 1 else 2
    es = kv_bytes(cfg)
    attn = (2 * d * q + 2 * d * kv) * wb
    if cfg.n_experts:
        ex = experts_per_layer if experts_per_layer is not None else min(cfg.n_experts, B * cfg.top_k)
        ffn = ex * 3 * d * f * wb + cfg.n_experts * d * wb
    else:
        ffn = 3 * d * f * wb
    head = V * d * wb
    return (L * (attn + ffn) + head + B * d * wb + L * 2 * kv * es * (readable + B) + B * V * 4)


def prefill_weight_bytes(cfg, P):
    """Weights one prefill of P tokens reads once (every expert a token chose;
    a P-token MoE prefill touches min(E, P*k) experts a layer)."""
    return decode_step_bytes(cfg, P, 0) - P * cfg.hidden * 2 - cfg.n_layers * 2 * cfg.kv_dim * kv_bytes(cfg) * P \
        - P * cfg.vocab * 4


def _hbm(bytes_, ms):
    ach = bytes_ / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "algorithmic_gb": round(bytes_ / 1e9, 4)}


def _kernel_roof(t, bound):
    if t["launches"] == 0 or t["ms"] <= 0:
        return None
    per = t["ms"] / t["launches"]
    if bound == "hbm":
        ach = t["bytes"] / t["launches"] / (per * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "avg_launch_us": round(per * 1e3, 2),
                "launches": t["launches"]}
    ach = t["flops"] / t["launches"] / (per * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(ach, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / BF16_PEAK_TFLOPS, 4), "avg_launch_us": round(per * 1e3, 2),
            "launches": t["launches"]}


def run_other(cfg, Bs, P, steps, warmup, phase="all"):
    """One shape's workload: prefill P tokens into each of max(Bs) slots, then
    batched greedy decode at each B in Bs (largest first; a smaller B reuses
    slots 0..B-1 after re-prefilling them, so it also starts at position P)."""
    import numpy as np
    import torch
    from decoder_only_forward_amd import synth
    from decoder_only_forward_amd import dec as D

    t0 = time.perf_counter()
    wd = synth.make_weights(cfg, seed=0, device="cuda")
    torch.cuda.synchronize()
    log(f"[{cfg.name}] weights {cfg.matrix_params() / 1e9:.2f} B params drawn in {time.perf_counter() - t0:.1f} s")
    Bmax = max(Bs)
    model = D.DecModel(cfg, wd, max_batch=Bmax, max_prefill=P)
    prompts = synth.prompts(cfg, Bmax, P)
    logits1 = torch.empty(cfg.vocab, device="cuda")
    out = {"workload": f"{cfg.name}: prefill P={P} into {Bmax} slots; decode B={'/'.join(map(str, Bs))} "
                       f"from position {P}", "layers": cfg.n_layers}

    model.timing_enable(D.DEC_K_GEMM)
    model.timing_enable(D.DEC_K_ATTN_PREFILL)
    pre_ms = []
    n_pre = Bmax if phase != "prefill" else min(Bmax, 3)
    for b in range(n_pre):
        torch.cuda.synchronize()
        t = time.perf_counter()
        model.prefill(prompts[b].tolist(), seq=b, logits=logits1)
        torch.cuda.synchronize()
        pre_ms.append((time.perf_counter() - t) * 1e3)
    gemm_t = model.timing_read(D.DEC_K_GEMM)
    apre_t = model.timing_read(D.DEC_K_ATTN_PREFILL)
    model.timing_enable(D.DEC_K_GEMM, False)
    model.timing_enable(D.DEC_K_ATTN_PREFILL, False)
    med = float(np.median(pre_ms[1:] if len(pre_ms) > 2 else pre_ms))
    pre = {"P": P, "calls": len(pre_ms), "ms": round(med, 3), "tok_s": round(P / (med * 1e-3), 1),
           "hbm": _hbm(prefill_weight_bytes(cfg, P), med),
           "roofline_kernels": {"gemm_prefill": _kernel_roof(gemm_t, "mfma"),
                                "attn_prefill": _kernel_roof(apre_t, "mfma")}}
    if not cfg.n_experts:
        # useful flops of the whole call: every layer's projections on P rows, the
        # LM head on the last row, causal attention (2 hd products per head and key)
        layer_params = cfg.matrix_params() - cfg.vocab * cfg.hidden * (1 if cfg.tied_embedding else 2)
        flops = 2.0 * P * layer_params + 2.0 * cfg.vocab * cfg.hidden + \
            cfg.n_layers * 2.0 * cfg.head_dim * cfg.n_heads * P * (P + 1)
        pre["mfma_useful_whole_call"] = round(flops / (med * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)
    out["prefill"] = pre
    log(f"[{cfg.name}] prefill P={P}: {med:.2f} ms median of {len(pre_ms)}, {P / (med * 1e-3):.0f} tok/s")
    if phase == "prefill":
        model.close()
        return out

    out["decode"] = {}
    for B in sorted(Bs, reverse=True):
        if B != Bmax:
            for b in range(B):
                model.reset(b)
                model.prefill(prompts[b].tolist(), seq=b, logits=logits1)
        lg = torch.empty((B, cfg.vocab), device="cuda")
        toks = np.asarray(synth.prompts(cfg, B, 1, stream=synth.TEACHER_STREAM)[:, 0], dtype=np.int32)
        experts = None
        if cfg.n_experts:
            # the experts one step's tokens choose (an eager step with the ids captured)
            ids = torch.zeros((cfg.n_layers, B, cfg.top_k), dtype=torch.int32, device="cuda")
            model.set_capture(None, ids, None)
            pos = np.array([model.length(b) for b in range(B)], dtype=np.int32)
            model.decode(toks, pos, logits=lg)
            toks[:] = model.greedy(lg, B)
            model.set_capture(None, None, None)
            ic = ids.cpu().numpy()
            experts = float(np.mean([len(np.unique(ic[l])) for l in range(cfg.n_layers)]))

        def step():
            pos = np.array([model.length(b) for b in range(B)], dtype=np.int32)
            model.decode(toks, pos, logits=lg)
            toks[:] = model.greedy(lg, B)
            return pos

        for _ in range(warmup):
            step()
        nbytes = 0.0
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(steps):
            pos = step()
            nbytes += decode_step_bytes(cfg, B, int(np.sum(np.minimum(pos + 1, cfg.max_seq))), experts)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t
        model.timing_enable(D.DEC_K_GEMV)
        model.timing_enable(D.DEC_K_ATTN_DECODE)
        for _ in range(steps):
            step()
        gemv_t = model.timing_read(D.DEC_K_GEMV)
        attn_t = model.timing_read(D.DEC_K_ATTN_DECODE)
        model.timing_enable(D.DEC_K_GEMV, False)
        model.timing_enable(D.DEC_K_ATTN_DECODE, False)
        ms = dt * 1e3 / steps
        r = {"tok_s": round(B * steps / dt, 2), "ms_per_step": round(ms, 4), "steps": steps,
             "roofline": _hbm(nbytes / steps, ms),
             "roofline_kernels": {"gemv_decode": _kernel_roof(gemv_t, "hbm"),
                                  "attn_decode": _kernel_roof(attn_t, "hbm")}}
        if experts is not None:
            r["experts_per_layer"] = round(experts, 3)
            r["note"] = ("step bytes count the experts the step's tokens chose; the GEMV object counts "
                         "min(E, B*k) experts a layer")
        out["decode"][f"b{B}"] = r
        log(f"[{cfg.name}] decode B={B}: {ms:.3f} ms/step, {B * steps / dt:.1f} tok/s, "
            f"{r['roofline']['frac'] * 100:.1f} % of HBM")
    model.close()
    del model, wd
    torch.cuda.empty_cache()
    return out


def run_prefill_only(cfg, wd, P, calls=3):
    """A few prefill calls of P tokens (for counter runs of the prefill kernels)."""
    import torch
    from decoder_only_forward_amd import synth
    from decoder_only_forward_amd import dec as D
    model = D.DecModel(cfg, wd, max_batch=1, max_prefill=P)
    prompt = synth.prompts(cfg, 1, P)[0].tolist()
    logits = torch.empty(cfg.vocab, device="cuda")
    for i in range(calls):
        model.reset()
        torch.cuda.synchronize()
        t = time.perf_counter()
        model.prefill(prompt, logits=logits)
        torch.cuda.synchronize()
        log(f"[{cfg.name}] prefill P={P} call {i}: {(time.perf_counter() - t) * 1e3:.1f} ms")
    model.close()


def run_prefill_variant(cfg, wd, P, calls=5):
    """Prefill calls of P tokens into one slot (the first call discarded): the
    median call time and the GEMM launches' timing."""
    import numpy as np
    import torch
    from decoder_only_forward_amd import synth
    from decoder_only_forward_amd import dec as D
    model = D.DecModel(cfg, wd, max_batch=1, max_prefill=P)
    prompt = synth.prompts(cfg, 1, P)[0].tolist()
    logits = torch.empty(cfg.vocab, device="cuda")
    ms = []
    for i in range(calls):
        model.reset()
        if i == 1:
            model.timing_enable(D.DEC_K_GEMM)
        torch.cuda.synchronize()
        t = time.perf_counter()
        model.prefill(prompt, logits=logits)
        torch.cuda.synchronize()
        ms.append((time.perf_counter() - t) * 1e3)
    gemm_t = model.timing_read(D.DEC_K_GEMM)
    model.close()
    del model
    torch.cuda.empty_cache()
    med = float(np.median(ms[1:]))
    log(f"[{cfg.name}] prefill P={P}: {med:.1f} ms median of {calls - 1}")
    return {"ms": med, "gemm": gemm_t}


def run_workload(cfg, wd, B, P, steps, warmup, small_batches=()):
    """Prefill P tokens into each of B slots, then time batched greedy decode."""
    import numpy as np
    import torch
    from decoder_only_forward_amd import synth
    from decoder_only_forward_amd import dec as D

    model = D.DecModel(cfg, wd, max_batch=B, max_prefill=P)
    kvname = kv_name(cfg)
    log(f"[{kvname} KV] workspace {model.workspace.numel() / 2**30:.1f} GiB")
    prompts = synth.prompts(cfg, B, P)

    # setup: prefill every slot; each call is a prefill sample
    logits1 = torch.empty(cfg.vocab, device="cuda")
    model.timing_enable(D.DEC_K_GEMM)
    model.timing_enable(D.DEC_K_ATTN_PREFILL)
    pre_ms = []
    for b in range(B):
        torch.cuda.synchronize()
        t = time.perf_counter()
        model.prefill(prompts[b].tolist(), seq=b, logits=logits1)
        torch.cuda.synchronize()
        pre_ms.append((time.perf_counter() - t) * 1e3)
        if b == 0:
            log(f"[{kvname} KV] prefill slot 0: {pre_ms[0]:.1f} ms")
    gemm_t = model.timing_read(D.DEC_K_GEMM)
    apre_t = model.timing_read(D.DEC_K_ATTN_PREFILL)
    model.timing_enable(D.DEC_K_GEMM, False)
    model.timing_enable(D.DEC_K_ATTN_PREFILL, False)
    pre_med = float(np.median(pre_ms))
    log(f"[{kvname} KV] prefill median {pre_med:.1f} ms over {B} calls")

    logits = torch.empty((B, cfg.vocab), device="cuda")
    nxt = model.greedy(logits1, 1)  # any valid tokens
    toks = np.full(B, int(nxt[0]), dtype=np.int32)

    def step():
        pos = np.array([model.length(b) for b in range(B)], dtype=np.int32)
        model.decode(toks, pos, logits=logits)
        toks[:] = model.greedy(logits, B)

    for _ in range(warmup):
        step()
    # timed region 1: throughput (decode steps replay a captured HIP graph)
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t
    ms_step = dt * 1e3 / steps
    value = B * steps / dt
    log(f"[{kvname} KV] decode B={B}: {ms_step:.2f} ms/step, {value:.1f} tok/s ({model.graph_count()} graphs)")
    # timed region 1b: the same steps as one device-resident greedy loop (the
    # choices feed the next step on the GPU; one graph replay per step)
    loop_logits = torch.empty((B, cfg.vocab), device="cuda")
    loop_out = torch.empty((steps, B), dtype=torch.int32, device="cuda")
    model.decode_greedy(toks, min(2, steps), logits=loop_logits, out=loop_out[:min(2, steps)])  # capture
    torch.cuda.synchronize()
    t = time.perf_counter()
    model.decode_greedy(toks, steps, logits=loop_logits, out=loop_out)
    torch.cuda.synchronize()
    dt_loop = time.perf_counter() - t
    toks[:] = loop_out[-1].cpu().numpy()
    log(f"[{kvname} KV] decode B={B} device loop: {dt_loop * 1e3 / steps:.2f} ms/step, {B * steps / dt_loop:.1f} tok/s")
    # timed region 2: the same steps with every GEMV and attention launch
    # bracketed by HIP events on the library's stream (eager launches)
    model.timing_enable(D.DEC_K_GEMV)
    model.timing_enable(D.DEC_K_ATTN_DECODE)
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    dt_timed = time.perf_counter() - t
    gemv_t = model.timing_read(D.DEC_K_GEMV)
    attn_t = model.timing_read(D.DEC_K_ATTN_DECODE)
    model.timing_enable(D.DEC_K_GEMV, False)
    model.timing_enable(D.DEC_K_ATTN_DECODE, False)
    log(f"[{kvname} KV] decode B={B} with kernel events (eager): {dt_timed * 1e3 / steps:.2f} ms/step")

    # smaller batches on the same cache (each row continues its own sequence)
    extra = {}
    for bb in small_batches:
        if bb >= B:
            continue
        lg = torch.empty((bb, cfg.vocab), device="cuda")
        tk = toks[:bb].copy()
        for _ in range(2):
            pos = np.array([model.length(b) for b in range(bb)], dtype=np.int32)
            model.decode(tk, pos, logits=lg)
            tk[:] = model.greedy(lg, bb)
        torch.cuda.synchronize()
        t = time.perf_counter()
        n = max(8, steps // 2)
        for _ in range(n):
            pos = np.array([model.length(b) for b in range(bb)], dtype=np.int32)
            model.decode(tk, pos, logits=lg)
            tk[:] = model.greedy(lg, bb)
        torch.cuda.synchronize()
        e = time.perf_counter() - t
        extra[f"b{bb}"] = {"tok_s": round(bb * n / e, 2), "ms_per_step": round(e * 1e3 / n, 3)}
        log(f"[{kvname} KV] decode B={bb}: {e * 1e3 / n:.2f} ms/step")
    # AppendPrefill past the ring's size in one pass (deferred commit): 512
    # tokens appended to slot 0, whose ring is already full
    append = None
    if cfg.sliding_window and cfg.max_seq == cfg.sliding_window:
        n_app = min(512, P)
        app = synth.prompts(cfg, 1, 3 * n_app, stream=synth.TEACHER_STREAM)[0].tolist()
        ms = []
        for i in range(3):
            torch.cuda.synchronize()
            t = time.perf_counter()
            model.prefill(app[i * n_app:(i + 1) * n_app], seq=0, start_pos=model.length(0), logits=logits1)
            torch.cuda.synchronize()
            ms.append((time.perf_counter() - t) * 1e3)
        med = float(np.median(ms))
        append = {"tokens": n_app, "ms": round(med, 2), "tok_s": round(n_app / (med * 1e-3), 1)}
        log(f"[{kvname} KV] append {n_app} tokens past the ring: {med:.1f} ms")
    model.close()
    del model
    torch.cuda.empty_cache()
    return {"value": value, "ms_step": ms_step, "pre_med": pre_med, "gemm": gemm_t, "apre": apre_t,
            "gemv": gemv_t, "attn": attn_t, "extra": extra, "dt_timed": dt_timed,
            "loop": {"tok_s": round(B * steps / dt_loop, 2), "ms_per_step": round(dt_loop * 1e3 / steps, 3)},
            "append": append}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=32)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--config", default="mistral-7b")
    ap.add_argument("--batch", type=int, default=32)
    ap.add_argument("--prompt", type=int, default=4096)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-steps", type=int, default=32, help="prompt tokens the oracle's prefill sample takes")
    ap.add_argument("--kv", choices=("all", "fp32", "f24"), default="all",
                    help="all: the fp32-cache run gives `value`; runs on a bf16 cache and on the 24-bit cache are "
                         "reported beside it.  fp32: only the fp32-cache run.  f24: only a 24-bit-cache run (with "
                         "--only mistral-7b, for profiling)")
    ap.add_argument("--pmc-calibration", action="store_true",
                    help="only run three 1 GiB device-to-device copies (PMC byte-counter calibration)")
    ap.add_argument("--only", choices=sorted(OTHER) + ["mistral-7b"], default=None,
                    help="run one workload alone and print its own JSON line (for profiling)")
    ap.add_argument("--phase", choices=("all", "prefill", "decode"), default="all",
                    help="with --only: stop after the prefill calls (a few of them) or run everything")
    ap.add_argument("--no-other", action="store_true", help="skip the other shapes' workloads")
    ap.add_argument("--layers", type=int, default=0,
                    help="with --only: keep this many layers (the per-layer shapes unchanged), e.g. for counter runs")
    ap.add_argument("--prefill-fp8", action="store_true",
                    help="with --only: prefill projections on fp16 + fp8 split operands (DEC_PREFILL_F16_F8) "
                         "instead of the bf16 pair")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (sharded, each GPU would "
              "serve its own sequences with its own copy of the weights and no exchange between GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from decoder_only_forward_amd import configs, synth
    from decoder_only_forward_amd import dec as D

    if args.pmc_calibration:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)  # one kernel: 1 GiB read, 1 GiB written
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read": 1 << 30, "bytes_written": 1 << 30, "launches": 3}))
        return

    torch.cuda.set_device(0)
    def shape(name):
        c = configs.CONFIGS[name]
        if args.only and args.layers > 0:
            c = c.replace(name=f"{c.name}-{args.layers}l", n_layers=args.layers)
        if args.only and args.prefill_fp8:
            c = c.replace(name=f"{c.name}-prefill-f16f8", prefill_fp8=True)
        if args.kv == "f24":
            c = c.replace(kv_f24=True)
        return c

    if args.only and args.only != "mistral-7b":
        Bs, P = OTHER[args.only]
        print(json.dumps(run_other(shape(args.only), Bs, P, args.steps, args.warmup, args.phase)), flush=True)
        return
    cfg = shape(args.only or args.config)
    B, P = args.batch, args.prompt
    t0 = time.perf_counter()
    wd = synth.make_weights(cfg, seed=0, device="cuda")
    torch.cuda.synchronize()
    log(f"weights {cfg.matrix_params() / 1e9:.2f} B params drawn in {time.perf_counter() - t0:.1f} s")

    if args.only == "mistral-7b" and args.phase == "prefill":
        run_prefill_only(cfg, wd, P)
        return
    main_run = run_workload(cfg, wd, B, P, args.steps, args.warmup, small_batches=(1, 8))
    bf16_run = f24_run = None
    if args.kv == "all" and not args.only:
        bf16_run = run_workload(cfg.replace(kv_bf16=True), wd, B, P, args.steps, args.warmup, small_batches=(1, 8))
        f24_run = run_workload(cfg.replace(kv_f24=True), wd, B, P, args.steps, args.warmup, small_batches=(1, 8))
    value, ms_step, pre_med = main_run["value"], main_run["ms_step"], main_run["pre_med"]
    gemm_t, apre_t, gemv_t, attn_t = main_run["gemm"], main_run["apre"], main_run["gemv"], main_run["attn"]
    extra, dt_timed = main_run["extra"], main_run["dt_timed"]

    def roof(t, bound, traffic_key=None, passes=None):
        if t["launches"] == 0 or t["ms"] <= 0:
            return None
        tr = measured_traffic(traffic_key, (cfg.name, B, P)) if traffic_key else None
        tr = None if tr is None else round(tr / 1e9, 4)
        per = t["ms"] / t["launches"]
        if bound == "hbm":
            ach = t["bytes"] / t["launches"] / (per * 1e-3) / 1e9
            return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": tr, "traffic_unit": "GB per launch (rocprofv3 PMC)",
                    "avg_launch_us": round(per * 1e3, 2), "launches": t["launches"]}
        ach = t["flops"] / t["launches"] / (per * 1e-3) / 1e12
        r = {"bound": "mfma", "achieved": round(ach, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
             "frac": round(ach / BF16_PEAK_TFLOPS, 4), "traffic": tr, "traffic_unit": "GB per launch (rocprofv3 PMC)",
             "avg_launch_us": round(per * 1e3, 2), "launches": t["launches"]}
        if passes:
            # achieved counts useful flops; each product runs as `passes` bf16
            # MFMA products (the fp32 operand split into a bf16 hi/lo pair)
            r["mfma_passes"] = passes
            r["executed_frac"] = round(passes * ach / BF16_PEAK_TFLOPS, 4)
            r["mfma_counters"] = measured_mfma(traffic_key, (cfg.name, B, P)) if traffic_key else None
        return r

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16 weights x fp32 (split-bf16 MFMA), " if not cfg.prefill_fp8 else
                  "bf16 weights x fp32 (decode: split-bf16 MFMA; prefill q|k|v and gate|up: fp16 + scaled fp8 "
                  "split operands), ") + {"fp32": "fp32 KV", "f24": "24-bit KV (16 significant bits)",
                                          "bf16": "bf16 KV"}[kv_name(cfg)],
        "data": "synthetic (seeded random-init weights and prompts)",
        "config": {"workload": f"{cfg.name} decode B={B} at positions {P}.. (ring KV {cfg.max_seq}), "
                               f"prefill P={P}", "batch": B, "prompt": P, "layers": cfg.n_layers},
        "prefill_tok_s": round(P / (pre_med * 1e-3), 1),
        "prefill_ms": round(pre_med, 2),
        "decode": extra,
        "decode_device_loop": main_run["loop"],
        "append_prefill_past_ring": main_run["append"],
        "ms_per_step_with_kernel_events": round(dt_timed * 1e3 / args.steps, 3),
        "roofline_kernels": {"gemv_decode": roof(gemv_t, "hbm", ("gemv_decode", "fp32")),
                             # (with fp16 + fp8 operands the launches mix 1.5- and 2-unit forms:
                             # no single pass count)
                             "gemm_prefill": roof(gemm_t, "mfma", ("gemm_prefill", "fp32"),
                                                  passes=None if cfg.prefill_fp8 else 2),
                             # hi*hi + hi*lo + lo*hi; causally masked halves of diagonal
                             # tiles run too, so the executed fraction is a lower bound
                             "attn_prefill": roof(apre_t, "mfma", ("attn_prefill", "fp32"), passes=3)},
    }

    def attn_roof(t, kv):
        # groups of up to 4 heads with an fp32 cache take the lane-group kernel,
        # the others the MFMA form
        name = ("attn_decode_kernel" if kv != "bf16" and cfg.n_heads // cfg.n_kv_heads <= 4
                else "attn_decode_mfma_kernel")
        r = roof(t, "hbm", (name, kv))
        if r is not None:
            r["kernel"] = f"{name} (split-KV GQA decode attention, {kv} KV)"
            r["algorithmic_bytes_per_launch_gb"] = round(t["bytes"] / t["launches"] / 1e9, 4)
        return r

    out["roofline"] = attn_roof(attn_t, kv_name(cfg))
    if bf16_run is not None:
        out["kv_bf16"] = {
            "note": "same workload with the K/V cache stored as nearest-even bf16 (arithmetic fp32)",
            "decode_tok_s": round(bf16_run["value"], 2),
            "ms_per_step": round(bf16_run["ms_step"], 3),
            "prefill_tok_s": round(P / (bf16_run["pre_med"] * 1e-3), 1),
            "prefill_ms": round(bf16_run["pre_med"], 2),
            "decode": bf16_run["extra"],
            "decode_device_loop": bf16_run["loop"],
            "append_prefill_past_ring": bf16_run["append"],
            "ms_per_step_with_kernel_events": round(bf16_run["dt_timed"] * 1e3 / args.steps, 3),
            "roofline": attn_roof(bf16_run["attn"], "bf16"),
            "roofline_kernels": {"gemv_decode": roof(bf16_run["gemv"], "hbm", ("gemv_decode", "bf16")),
                                 "attn_prefill": roof(bf16_run["apre"], "mfma", passes=2)},
        }
    if f24_run is not None:
        out["kv_f24"] = {
            "note": ("same workload with the K/V cache stored at 16 significant bits (fp32 rounded to nearest "
                     "even at 15 stored mantissa bits, 3 bytes an element; arithmetic fp32); parity-tested at "
                     "the fp32 cache's tolerances, also against the fp32-cache oracle"),
            "decode_tok_s": round(f24_run["value"], 2),
            "ms_per_step": round(f24_run["ms_step"], 3),
            "prefill_tok_s": round(P / (f24_run["pre_med"] * 1e-3), 1),
            "prefill_ms": round(f24_run["pre_med"], 2),
            "decode": f24_run["extra"],
            "decode_device_loop": f24_run["loop"],
            "append_prefill_past_ring": f24_run["append"],
            "ms_per_step_with_kernel_events": round(f24_run["dt_timed"] * 1e3 / args.steps, 3),
            "roofline": attn_roof(f24_run["attn"], "f24"),
            "roofline_kernels": {"gemv_decode": roof(f24_run["gemv"], "hbm", ("gemv_decode", "f24")),
                                 "attn_prefill": roof(f24_run["apre"], "mfma", passes=3)},
        }
    if args.kv == "all" and not args.only and not cfg.prefill_fp8:
        # the same prefill with the q|k|v and gate|up projections on fp16 + fp8
        # split operands (opt-in DEC_PREFILL_F16_F8), next to the bf16 pair's
        # prefill on the same model slot
        pv = run_prefill_variant(cfg.replace(name=cfg.name + "-prefill-f16f8", prefill_fp8=True), wd, P)
        pb = run_prefill_variant(cfg, wd, P)
        out["prefill_f16f8"] = {
            "note": ("prefill with q|k|v and gate|up as an fp16 pass plus a scaled fp8 pass (the weights' "
                     "upper bytes as e5m2 against the activation's fp8 remainder), o and down on the bf16 "
                     "pair; parity-tested at the fp32 path's tolerances; one slot, median of 4 calls, with "
                     "the bf16 pair timed the same way beside it"),
            "prefill_ms": round(pv["ms"], 2), "prefill_tok_s": round(P / (pv["ms"] * 1e-3), 1),
            "bf16_pair_prefill_ms": round(pb["ms"], 2),
            "gemm_prefill": roof(pv["gemm"], "mfma"),
            "gemm_prefill_bf16_pair": roof(pb["gemm"], "mfma"),
        }
        if out["prefill_f16f8"]["gemm_prefill"] is not None:
            out["prefill_f16f8"]["gemm_prefill"]["mfma_counters"] = measured_mfma(("gemm_prefill_f16f8", "fp32"),
                                                                                  (cfg.name, B, P))
    if not args.only:
        # measured ceilings beside the published peaks the roofline objects use
        out["ceilings"] = ceilings()
        out["roofline"]["frac_of_measured_read"] = round(out["roofline"]["achieved"] /
                                                         out["ceilings"]["hbm_read_GBps"], 4)
    if not args.no_cpu_baseline and not args.only:
        try:
            out["cpu_baseline"] = cpu_baseline(cfg, wd, B=B, prefill_tokens=args.cpu_steps)
        except Exception as e:  # the host may lack memory for the weights
            out["cpu_baseline"] = {"value": None, "error": str(e)}
    if not args.no_other and not args.only:
        del wd
        torch.cuda.empty_cache()
        out["workloads"] = {}
        for name in ("smollm2-135m", "qwen2.5-0.5b", "mixtral-8x7b"):
            Bs, Pn = OTHER[name]
            out["workloads"][name] = run_other(configs.CONFIGS[name], Bs, Pn, args.steps, args.warmup)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
