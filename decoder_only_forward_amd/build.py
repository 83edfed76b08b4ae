"""Build libdec.so (the HIP library) and libdec_probe.so (the measured-ceiling
probes) for gfx950 with hipcc, in-tree.

    python -m decoder_only_forward_amd.build

Every source is compiled on every call (the build check), in parallel.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "libdec.so")
OUT_PROBE = os.path.join(HERE, "libdec_probe.so")
OBJDIR = os.path.join(HERE, "_build")
SOURCES = ["k_elementwise.hip", "k_gemv.hip", "k_gemm.hip", "k_attn_decode.hip", "k_attn_prefill.hip", "k_attn_prefill_tiles.hip", "k_moe.hip", "dec_api.hip"]
PROBE_SOURCES = ["probe_ceilings.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-fvisibility=hidden",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], OUT)
    _link(objs[len(SOURCES):], OUT_PROBE)
    if verbose:
        print(f"built {OUT} and {OUT_PROBE}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
