"""Thin ctypes binding of libdec.so (include/dec.h): argument marshalling only.

Every step of the forward runs in the library's HIP kernels.  PyTorch provides
device memory (weights, workspace, logits) and the stream.  If the library has
not been built, `load()` raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

from .configs import ModelConfig, WEIGHT_F32

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdec.so")

DEC_OK, DEC_ERR_INVALID, DEC_ERR_RANGE, DEC_ERR_NOMEM, DEC_ERR_DEVICE, DEC_ERR_UNSUPPORTED = 0, -1, -2, -3, -4, -5
DEC_KV_F32, DEC_KV_BF16, DEC_KV_F24 = 0, 1, 2
DEC_K_GEMV, DEC_K_ATTN_DECODE, DEC_K_GEMM, DEC_K_ATTN_PREFILL = 0, 1, 2, 3
DEC_NOALLOC_WORKSPACE_BYTES = 64 << 20
EXPORTS = ("dec_workspace_bytes", "dec_create", "dec_create_noalloc", "dec_destroy", "dec_prefill", "dec_prefill_ex", "dec_decode",
           "dec_decode_greedy", "dec_kv_reset",
           "dec_graph_count", "dec_kv_length", "dec_greedy", "dec_sync", "dec_set_capture", "dec_timing_enable",
           "dec_timing_read", "dec_status_str")


class DecConfig(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32)] + [(n, ctypes.c_int32) for n in (
        "n_layers", "hidden", "n_heads", "n_kv_heads", "head_dim", "ffn_dim", "vocab", "n_experts", "top_k",
        "qkv_bias", "tied_embedding", "sliding_window", "max_seq", "max_batch", "max_prefill",
        "weight_dtype")] + [("rms_eps", ctypes.c_double), ("rope_theta", ctypes.c_double)] + [
        (n, ctypes.c_int32) for n in ("rope_pairing", "rope_scaling", "rope_orig_ctx", "kv_dtype")] + [
        (n, ctypes.c_double) for n in ("rope_factor", "rope_low_freq_factor", "rope_high_freq_factor")] + [
        ("prefill_operands", ctypes.c_int32)]


class DecLayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "attn_norm", "wq", "wk", "wv", "bq", "bk", "bv", "wo", "ffn_norm", "w_gate", "w_up", "w_down", "router")]


class DecWeights(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("embed", ctypes.c_void_p), ("out_norm", ctypes.c_void_p),
                ("lm_head", ctypes.c_void_p), ("layers", ctypes.POINTER(DecLayerWeights))]


class DecError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        msg = _lib.dec_status_str(code).decode() if _lib is not None else str(code)
        super().__init__(f"{what}: {msg} ({code})")
        self.code = code


_lib = None


def load():
    """Open libdec.so; raise if it is missing (build with
    `python -m decoder_only_forward_amd.build`)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m decoder_only_forward_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, c_int = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int
    L.dec_workspace_bytes.restype = ctypes.c_size_t
    L.dec_workspace_bytes.argtypes = [ctypes.POINTER(DecConfig)]
    L.dec_create.restype = c_int
    L.dec_create.argtypes = [ctypes.POINTER(DecConfig), ctypes.POINTER(DecWeights), vp, ctypes.c_size_t, vp,
                             ctypes.POINTER(vp)]
    L.dec_create_noalloc.restype = c_int
    L.dec_create_noalloc.argtypes = [ctypes.POINTER(DecConfig), ctypes.POINTER(DecWeights), vp, ctypes.POINTER(vp)]
    L.dec_destroy.restype = None
    L.dec_destroy.argtypes = [vp]
    L.dec_prefill.restype = c_int
    L.dec_prefill.argtypes = [vp, c_int, vp, c_int, c_int, vp]
    L.dec_prefill_ex.restype = c_int
    L.dec_prefill_ex.argtypes = [vp, c_int, vp, c_int, c_int, vp, c_int]
    L.dec_decode.restype = c_int
    L.dec_decode.argtypes = [vp, c_int, vp, vp, vp]
    L.dec_decode_greedy.restype = c_int
    L.dec_decode_greedy.argtypes = [vp, c_int, vp, c_int, vp, vp]
    L.dec_kv_reset.restype = c_int
    L.dec_kv_reset.argtypes = [vp, c_int]
    L.dec_kv_length.restype = c_int
    L.dec_kv_length.argtypes = [vp, c_int]
    L.dec_greedy.restype = c_int
    L.dec_greedy.argtypes = [vp, vp, c_int, vp]
    L.dec_sync.restype = c_int
    L.dec_sync.argtypes = [vp]
    L.dec_set_capture.restype = c_int
    L.dec_set_capture.argtypes = [vp, vp, vp, vp]
    L.dec_timing_enable.restype = c_int
    L.dec_timing_enable.argtypes = [vp, c_int, c_int]
    L.dec_timing_read.restype = c_int
    L.dec_timing_read.argtypes = [vp, c_int, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64),
                                  ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    L.dec_graph_count.restype = c_int
    L.dec_graph_count.argtypes = [vp]
    L.dec_status_str.restype = ctypes.c_char_p
    L.dec_status_str.argtypes = [c_int]
    _lib = L
    return L


def kv_dtype(cfg: ModelConfig) -> int:
    """dec_config.kv_dtype of a config: DEC_KV_F32, DEC_KV_BF16 or DEC_KV_F24."""
    if getattr(cfg, "kv_f24", False):
        return DEC_KV_F24
    return DEC_KV_BF16 if cfg.kv_bf16 else DEC_KV_F32


def make_config(cfg: ModelConfig, max_batch: int, max_prefill: int, max_seq: Optional[int] = None) -> DecConfig:
    return DecConfig(ctypes.sizeof(DecConfig), cfg.n_layers, cfg.hidden, cfg.n_heads, cfg.n_kv_heads,
                     cfg.head_dim, cfg.ffn_dim, cfg.vocab, cfg.n_experts, cfg.top_k, int(cfg.qkv_bias),
                     int(cfg.tied_embedding), cfg.sliding_window, cfg.max_seq if max_seq is None else max_seq,
                     max_batch, max_prefill, 1 if cfg.weight_dtype == WEIGHT_F32 else 0, cfg.rms_eps,
                     cfg.rope_theta, cfg.rope_pairing, cfg.rope_scaling, cfg.rope_orig_ctx, kv_dtype(cfg),
                     cfg.rope_factor, cfg.rope_low_freq_factor, cfg.rope_high_freq_factor,
                     int(getattr(cfg, "prefill_fp8", False)))


def workspace_bytes(cfg: ModelConfig, max_batch: int, max_prefill: int, max_seq: Optional[int] = None) -> int:
    c = make_config(cfg, max_batch, max_prefill, max_seq)
    return load().dec_workspace_bytes(ctypes.byref(c))


def _i32(a) -> np.ndarray:
    if isinstance(a, torch.Tensor):
        a = a.cpu().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _dptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    assert t.is_cuda and t.is_contiguous()
    return t.data_ptr()


class DecModel:
    """One model bound to device weights (dict from synth.make_weights on
    cuda), with its own workspace and KV cache of `max_batch` sequence slots.
    noalloc=True makes the handle with dec_create_noalloc: the workspace is the
    library's own device array and nothing is allocated here."""

    def __init__(self, cfg: ModelConfig, weights: dict, max_batch: int = 1, max_prefill: int = 1,
                 max_seq: Optional[int] = None, stream: Optional[torch.cuda.Stream] = None,
                 noalloc: bool = False):
        self.L = load()
        self.cfg = cfg
        self.w = weights
        self.max_batch = max_batch
        self.ccfg = make_config(cfg, max_batch, max_prefill, max_seq)
        nbytes = self.L.dec_workspace_bytes(ctypes.byref(self.ccfg))
        if nbytes == 0:
            raise DecError(DEC_ERR_INVALID, "dec_workspace_bytes")
        self.workspace = None if noalloc else torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        layers = (DecLayerWeights * cfg.n_layers)()
        for i, lw in enumerate(weights["layers"]):
            for f, _ in DecLayerWeights._fields_:
                setattr(layers[i], f, _dptr(lw.get(f)))
        self._layers = layers
        self.cw = DecWeights(ctypes.sizeof(DecWeights), _dptr(weights["embed"]), _dptr(weights["out_norm"]),
                             _dptr(weights["lm_head"]), layers)
        h = ctypes.c_void_p()
        if noalloc:
            rc = self.L.dec_create_noalloc(ctypes.byref(self.ccfg), ctypes.byref(self.cw),
                                           ctypes.c_void_p(self.stream.cuda_stream), ctypes.byref(h))
        else:
            rc = self.L.dec_create(ctypes.byref(self.ccfg), ctypes.byref(self.cw), _dptr(self.workspace), nbytes,
                                   ctypes.c_void_p(self.stream.cuda_stream), ctypes.byref(h))
        if rc != DEC_OK:
            raise DecError(rc, "dec_create_noalloc" if noalloc else "dec_create")
        self.h = h

    def close(self):
        if getattr(self, "h", None):
            self.L.dec_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check(self, rc: int, what: str):
        if rc != DEC_OK:
            raise DecError(rc, what)

    def prefill(self, tokens: Sequence[int], seq: int = 0, start_pos: int = 0,
                logits: Optional[torch.Tensor] = None, all_logits: bool = False) -> torch.Tensor:
        """Logits of the last position [vocab], or of every position [n, vocab]."""
        tok = _i32(tokens)
        if logits is None:
            shape = (tok.size, self.cfg.vocab) if all_logits else (self.cfg.vocab,)
            logits = torch.empty(shape, dtype=torch.float32, device="cuda")
        if all_logits:
            rc = self.L.dec_prefill_ex(self.h, seq, tok.ctypes.data, tok.size, start_pos, _dptr(logits), 1)
        else:
            rc = self.L.dec_prefill(self.h, seq, tok.ctypes.data, tok.size, start_pos, _dptr(logits))
        self._check(rc, "dec_prefill")
        return logits

    def decode(self, tokens: Sequence[int], pos: Sequence[int],
               logits: Optional[torch.Tensor] = None) -> torch.Tensor:
        tok, ps = _i32(tokens), _i32(pos)
        if logits is None:
            logits = torch.empty((tok.size, self.cfg.vocab), dtype=torch.float32, device="cuda")
        self._check(self.L.dec_decode(self.h, tok.size, tok.ctypes.data, ps.ctypes.data, _dptr(logits)),
                    "dec_decode")
        return logits

    def decode_greedy(self, tokens: Sequence[int], steps: int, logits: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None):
        """`steps` greedy steps on the device from tokens[b] at each row's length.
        Returns (choices [steps, B] int32 on the device, logits [B, vocab])."""
        tok = _i32(tokens)
        if logits is None:
            logits = torch.empty((tok.size, self.cfg.vocab), dtype=torch.float32, device="cuda")
        if out is None:
            out = torch.empty((steps, tok.size), dtype=torch.int32, device="cuda")
        self._check(self.L.dec_decode_greedy(self.h, tok.size, tok.ctypes.data, steps, _dptr(out), _dptr(logits)),
                    "dec_decode_greedy")
        return out, logits

    def greedy(self, logits: torch.Tensor, B: int) -> np.ndarray:
        out = np.empty(B, dtype=np.int32)
        self._check(self.L.dec_greedy(self.h, _dptr(logits), B, out.ctypes.data), "dec_greedy")
        return out

    def reset(self, seq: int = -1):
        self._check(self.L.dec_kv_reset(self.h, seq), "dec_kv_reset")

    def length(self, seq: int) -> int:
        r = self.L.dec_kv_length(self.h, seq)
        if r < 0:
            raise DecError(r, "dec_kv_length")
        return r

    def graph_count(self) -> int:
        return self.L.dec_graph_count(self.h)

    def sync(self):
        self._check(self.L.dec_sync(self.h), "dec_sync")

    def set_capture(self, hidden: Optional[torch.Tensor] = None, ids: Optional[torch.Tensor] = None,
                    router: Optional[torch.Tensor] = None):
        self._capture = (hidden, ids, router)
        self._check(self.L.dec_set_capture(self.h, _dptr(hidden), _dptr(ids), _dptr(router)), "dec_set_capture")

    def timing_enable(self, kernel_class: int, on: bool = True):
        self._check(self.L.dec_timing_enable(self.h, kernel_class, int(on)), "dec_timing_enable")

    def timing_read(self, kernel_class: int) -> dict:
        ms, n = ctypes.c_double(), ctypes.c_int64()
        b, f = ctypes.c_double(), ctypes.c_double()
        self._check(self.L.dec_timing_read(self.h, kernel_class, ctypes.byref(ms), ctypes.byref(n), ctypes.byref(b),
                                           ctypes.byref(f)), "dec_timing_read")
        return {"ms": ms.value, "launches": n.value, "bytes": b.value, "flops": f.value}
