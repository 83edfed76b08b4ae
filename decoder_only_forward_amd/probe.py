"""ctypes binding of libdec_probe.so (include/dec_probe.h): measured ceilings
for the roofline figures.  Argument marshalling only; the probes run in the
library's HIP kernels."""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdec_probe.so")
EXPORTS = ("decp_stream_read", "decp_copy", "decp_mfma_sink_floats", "decp_mfma_bf16")
RUN_BYTES = 16384   # DECP_RUN_BYTES

_lib = None


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, ci, dp = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.POINTER(ctypes.c_double)
        L.decp_mfma_sink_floats.restype = ci
        L.decp_mfma_sink_floats.argtypes = []
        L.decp_stream_read.restype = ci
        L.decp_stream_read.argtypes = [vp, sz, vp, ci, vp, dp]
        L.decp_copy.restype = ci
        L.decp_copy.argtypes = [vp, vp, sz, ci, vp, dp]
        L.decp_mfma_bf16.restype = ci
        L.decp_mfma_bf16.argtypes = [ci, vp, ci, vp, dp, dp]
        _lib = L
    return _lib


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what} failed ({rc})")


def stream_read(buf: torch.Tensor, reps: int = 5, sink: torch.Tensor | None = None) -> float:
    """Mean ms to read every byte of `buf` once (its byte size a multiple of
    RUN_BYTES); sink: one 32-bit word per RUN_BYTES run."""
    L = load()
    n = buf.numel() * buf.element_size()
    sink = torch.empty(n // RUN_BYTES, dtype=torch.int32, device="cuda") if sink is None else sink
    assert sink.numel() * sink.element_size() >= 4 * (n // RUN_BYTES)
    ms = ctypes.c_double()
    st = torch.cuda.current_stream().cuda_stream
    _check(L.decp_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(), reps, st,
                              ctypes.byref(ms)), "decp_stream_read")
    return ms.value


def copy(src: torch.Tensor, dst: torch.Tensor, reps: int = 5) -> float:
    """Mean ms to copy src into dst (same byte size)."""
    L = load()
    n = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() >= n
    ms = ctypes.c_double()
    st = torch.cuda.current_stream().cuda_stream
    _check(L.decp_copy(src.data_ptr(), dst.data_ptr(), n, reps, st, ctypes.byref(ms)), "decp_copy")
    return ms.value


def mfma_bf16(iters: int = 4096, reps: int = 5) -> tuple[float, float]:
    """(mean ms, flops) of one launch of the bf16 MFMA loop."""
    L = load()
    sink = torch.empty(L.decp_mfma_sink_floats(), dtype=torch.float32, device="cuda")
    ms, fl = ctypes.c_double(), ctypes.c_double()
    st = torch.cuda.current_stream().cuda_stream
    _check(L.decp_mfma_bf16(iters, sink.data_ptr(), reps, st, ctypes.byref(ms), ctypes.byref(fl)), "decp_mfma_bf16")
    return ms.value, fl.value
