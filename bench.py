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

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config mistral-7b]
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
           "34608c55f95e88c4c9dc0713feb1c89be769be0a7ff3031fa8e6327276c4082b"}
_ATTN_SOURCES = dict(_COMMON, **{"decoder_only_forward_amd/csrc/k_attn_decode.hip":
                                 "ca3d86f7b73f35f0be29369ea8bd3a6fb1fe27407b3b434c02588de0564dae0e"})
_GEMV_SOURCES = dict(_COMMON, **{"decoder_only_forward_amd/csrc/k_gemv.hip":
                                 "e8b40692db620676cb8b5a5653b879158cc66c2d689ff00d7afbbe436a81511c"})
_GEMM_SOURCES = dict(_COMMON, **{"decoder_only_forward_amd/csrc/k_gemm.hip":
                                 "2b5a11a5b66d407bcf10b64d4014b202650f0e067b23c57659c2175110e22eee"})
MEASURED_TRAFFIC = {
    ("attn_decode_kernel", "fp32"): {"sources": _ATTN_SOURCES, "workload": ("mistral-7b", 32, 4096),
                                     "bytes_per_launch": 1078815360},
    ("attn_decode_kernel", "bf16"): {"sources": _ATTN_SOURCES, "workload": ("mistral-7b", 32, 4096),
                                     "bytes_per_launch": 545073204},
    ("gemv_decode", "fp32"): {"sources": _GEMV_SOURCES, "workload": ("mistral-7b", 32, 4096),
                              "bytes_per_launch": 121762993},
    ("gemv_decode", "bf16"): {"sources": _GEMV_SOURCES, "workload": ("mistral-7b", 32, 4096),
                              "bytes_per_launch": 121762993},
    ("gemm_prefill", "fp32"): {"sources": _GEMM_SOURCES, "workload": ("mistral-7b", 32, 4096),
                               "bytes_per_launch": 1698152177},
}
BF16_PEAK_TFLOPS = 2500.0
METRIC = "decode tok/s + prefill tok/s (Mistral-7B shape) and % of HBM / MFMA roofline"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(kernel, workload):
    """kernel: (name, cache type); workload: (config name, batch, prompt)."""
    import hashlib
    m = MEASURED_TRAFFIC.get(kernel)
    if not m or m["workload"] != workload:
        return None
    for rel, sha in m["sources"].items():
        with open(os.path.join(ROOT, rel), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != sha:
                return None
    return m["bytes_per_launch"]


def cpu_baseline(cfg, wd, steps=4):
    """The oracle, untuned, on the host cores: greedy decode at B = 1 from an
    empty cache (positions 0..steps-1) on the same model (weights copied to host)."""
    import numpy as np
    from oracle import oracle as O
    O.build(force=False)
    w = {k: (v.cpu() if v is not None else None) for k, v in wd.items() if k != "layers"}
    w["layers"] = [{k: v.cpu() for k, v in lw.items()} for lw in wd["layers"]]
    ora = O.OracleModel(cfg, w, n_slots=1, max_seq=cfg.max_seq)
    tok = 1
    t0 = time.perf_counter()
    for p in range(steps):
        r = ora.decode([tok], [p])
        tok = int(np.argmax(r["logits"][0]))
    dt = time.perf_counter() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": steps / dt, "unit": "tok/s", "cores": threads, "kind": "oracle",
            "sample": f"{cfg.name} full depth, decode B=1 at positions 0..{steps - 1} "
                      f"({dt:.1f} s; the context is short, attention is <1% of the per-token work)"}


def run_workload(cfg, wd, B, P, steps, warmup, small_batches=()):
    """Prefill P tokens into each of B slots, then time batched greedy decode."""
    import numpy as np
    import torch
    from decoder_only_forward_amd import synth
    from decoder_only_forward_amd import dec as D

    model = D.DecModel(cfg, wd, max_batch=B, max_prefill=P)
    kvname = "bf16" if cfg.kv_bf16 else "fp32"
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
    ap.add_argument("--cpu-steps", type=int, default=32)
    ap.add_argument("--kv", choices=("both", "fp32"), default="both",
                    help="both: the fp32-cache run gives `value`, a bf16-cache run is reported beside it")
    ap.add_argument("--pmc-calibration", action="store_true",
                    help="only run three 1 GiB device-to-device copies (PMC byte-counter calibration)")
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

    cfg = configs.CONFIGS[args.config]
    B, P = args.batch, args.prompt
    torch.cuda.set_device(0)
    t0 = time.perf_counter()
    wd = synth.make_weights(cfg, seed=0, device="cuda")
    torch.cuda.synchronize()
    log(f"weights {cfg.matrix_params() / 1e9:.2f} B params drawn in {time.perf_counter() - t0:.1f} s")

    main_run = run_workload(cfg, wd, B, P, args.steps, args.warmup, small_batches=(1, 8))
    bf16_run = None
    if args.kv == "both":
        bf16_run = run_workload(cfg.replace(kv_bf16=True), wd, B, P, args.steps, args.warmup, small_batches=(1, 8))
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
        "dtype": "bf16 weights x fp32 (split-bf16 MFMA), fp32 KV",
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
                             "gemm_prefill": roof(gemm_t, "mfma", ("gemm_prefill", "fp32"), passes=2),
                             # hi*hi + hi*lo + lo*hi; causally masked halves of diagonal
                             # tiles run too, so the executed fraction is a lower bound
                             "attn_prefill": roof(apre_t, "mfma", passes=3)},
    }

    def attn_roof(t, kv):
        r = roof(t, "hbm", ("attn_decode_kernel", kv))
        if r is not None:
            r["kernel"] = f"attn_decode_kernel (split-KV GQA decode attention, {kv} KV)"
            r["algorithmic_bytes_per_launch_gb"] = round(t["bytes"] / t["launches"] / 1e9, 4)
        return r

    out["roofline"] = attn_roof(attn_t, "fp32")
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
    if not args.no_cpu_baseline:
        try:
            out["cpu_baseline"] = cpu_baseline(cfg, wd, args.cpu_steps)
        except Exception as e:  # the host may lack memory for the weights
            out["cpu_baseline"] = {"value": None, "error": str(e)}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
