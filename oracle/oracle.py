"""ctypes binding of the CPU oracle (oracle.c).  TEST INFRASTRUCTURE ONLY:
tests, the smoke check and the bench's CPU baseline use it; the product path
never imports it.

The oracle is built twice from the same C file: `f32` (fp32 arithmetic, the
oracle proper) and `f64` (its float64 shadow).  `build()` compiles both with
gcc; `OracleModel` wraps one model instance with its own KV cache.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
# ORACLE_LIB_DIR puts the built libraries elsewhere (a test that builds an
# instrumented copy uses it); ORACLE_SANITIZE=address builds them with the
# host compiler's AddressSanitizer (the process must preload libasan).
_LIB_DIR = os.environ.get("ORACLE_LIB_DIR", HERE)
LIBS = {"f32": os.path.join(_LIB_DIR, "liboracle32.so"), "f64": os.path.join(_LIB_DIR, "liboracle64.so")}
# Plain IEEE arithmetic: no FMA contraction, no fast-math, no target-specific ISA.
CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-fvisibility=hidden", "-lm"]
if os.environ.get("ORACLE_SANITIZE") == "address":
    CFLAGS = CFLAGS + ["-g", "-fno-omit-frame-pointer", "-fsanitize=address"]


def build(force: bool = True) -> None:
    for kind, out in LIBS.items():
        if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(SRC):
            continue
        defs = ["-DREAL=double", "-DORACLE_DOUBLE"] if kind == "f64" else ["-DREAL=float"]
        tmp = out + ".tmp"
        subprocess.check_call(["gcc", *defs, SRC, "-o", tmp, *CFLAGS])
        os.replace(tmp, out)


class OCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "hidden", "n_heads", "n_kv_heads", "head_dim", "ffn_dim", "vocab",
        "n_experts", "top_k", "qkv_bias", "sliding_window", "max_seq", "n_slots", "weight_f32",
        "window_by_mask")] + [("rms_eps", ctypes.c_double), ("rope_theta", ctypes.c_double)] + [
        (n, ctypes.c_int32) for n in ("rope_pairing", "rope_scaling", "rope_orig_ctx", "kv_round")] + [
        (n, ctypes.c_double) for n in ("rope_factor", "rope_low_freq_factor", "rope_high_freq_factor")]


class OLayer(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "attn_norm", "wq", "wk", "wv", "bq", "bk", "bv", "wo", "ffn_norm",
        "w_gate", "w_up", "w_down", "router")]


_loaded = {}


def kv_round(cfg) -> int:
    """Rounding of K/V at store: 0 none, 1 bf16, 2 the 24-bit float."""
    if getattr(cfg, "kv_f24", False):
        return 2
    return 1 if getattr(cfg, "kv_bf16", False) else 0


def lib(kind: str = "f32"):
    if kind not in _loaded:
        if not os.path.exists(LIBS[kind]) or os.path.getmtime(LIBS[kind]) < os.path.getmtime(SRC):
            build(force=False)
        L = ctypes.CDLL(LIBS[kind])
        pre = "oracle32_" if kind == "f32" else "oracle64_"
        for name, res in (("create", ctypes.c_void_p), ("destroy", None), ("reset", ctypes.c_int),
                          ("prefill", ctypes.c_int), ("decode", ctypes.c_int),
                          ("length", ctypes.c_int), ("argmax", ctypes.c_int),
                          ("rmsnorm", None), ("rope", None), ("moe_route", None),
                          ("attention_prefill", None), ("kv_row", None), ("rope_ex", None),
                          ("llama3_inv_freq", ctypes.c_double)):
            f = getattr(L, pre + name)
            f.restype = res
            setattr(L, name, f)
        L.create.argtypes = [ctypes.POINTER(OCfg), ctypes.c_void_p, ctypes.c_void_p,
                             ctypes.c_void_p, ctypes.POINTER(OLayer)]
        L.destroy.argtypes = [ctypes.c_void_p]
        L.reset.argtypes = [ctypes.c_void_p, ctypes.c_int]
        L.length.argtypes = [ctypes.c_void_p, ctypes.c_int]
        L.prefill.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                              ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.decode.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.argmax.argtypes = [ctypes.c_void_p, ctypes.c_int]
        L.rmsnorm.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_double,
                              ctypes.c_void_p]
        L.rope.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double]
        L.moe_route.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                ctypes.c_void_p]
        L.attention_prefill.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 5 + [ctypes.c_void_p]
        L.kv_row.argtypes = [ctypes.c_void_p] + [ctypes.c_int] * 4 + [ctypes.c_void_p]
        L.rope_ex.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                              ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                              ctypes.c_int]
        L.llama3_inv_freq.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                      ctypes.c_int]
        _loaded[kind] = L
    return _loaded[kind]


def np_dtype(kind: str):
    return np.float32 if kind == "f32" else np.float64


def _ptr(a) -> Optional[int]:
    if a is None:
        return None
    if isinstance(a, torch.Tensor):
        assert a.device.type == "cpu" and a.is_contiguous()
        return a.data_ptr()
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# ---- single ops (for the pins) -------------------------------------------

def rmsnorm(x, g, eps, kind="f32"):
    dt = np_dtype(kind)
    x = np.ascontiguousarray(x, dtype=dt)
    g = np.ascontiguousarray(g, dtype=np.float32)
    out = np.empty_like(x)
    lib(kind).rmsnorm(_ptr(x), _ptr(g), x.size, eps, _ptr(out))
    return out


def rope(h, n_heads, hd, pos, theta, kind="f32"):
    dt = np_dtype(kind)
    h = np.array(h, dtype=dt, order="C", copy=True)
    lib(kind).rope(_ptr(h), n_heads, hd, pos, theta)
    return h


def rope_ex(h, n_heads, hd, pos, theta, pairing=0, scaling=0, factor=8.0, low=1.0, high=4.0, orig_ctx=8192,
            kind="f32"):
    dt = np_dtype(kind)
    h = np.array(h, dtype=dt, order="C", copy=True)
    lib(kind).rope_ex(_ptr(h), n_heads, hd, pos, theta, pairing, scaling, factor, low, high, orig_ctx)
    return h


def llama3_inv_freq(f, factor, low, high, orig_ctx, kind="f64"):
    return lib(kind).llama3_inv_freq(f, factor, low, high, orig_ctx)


def moe_route(logits, k, kind="f32"):
    dt = np_dtype(kind)
    logits = np.ascontiguousarray(logits, dtype=dt)
    ids = np.empty(k, dtype=np.int32)
    w = np.empty(k, dtype=dt)
    lib(kind).moe_route(_ptr(logits), logits.size, k, _ptr(ids), _ptr(w))
    return ids, w


def attention_prefill(q, k, v, window=0, kind="f32"):
    """q [n, nh, hd], k/v [n, nkv, hd] -> o [n, nh, hd] (causal, optional window)."""
    dt = np_dtype(kind)
    q = np.ascontiguousarray(q, dtype=dt)
    k = np.ascontiguousarray(k, dtype=dt)
    v = np.ascontiguousarray(v, dtype=dt)
    n, nh, hd = q.shape
    out = np.empty_like(q)
    lib(kind).attention_prefill(_ptr(q), _ptr(k), _ptr(v), n, nh, k.shape[1], hd, window, _ptr(out))
    return out


# ---- model ---------------------------------------------------------------

class OracleError(RuntimeError):
    def __init__(self, code):
        super().__init__(f"oracle status {code}")
        self.code = code


class OracleModel:
    """One oracle model with `n_slots` sequence slots.  `weights` is the dict
    made by synth.make_weights (CPU tensors); they are borrowed and kept alive."""

    def __init__(self, cfg, weights, n_slots: int = 1, kind: str = "f32",
                 window_by_mask: bool = False, max_seq: Optional[int] = None):
        self.cfg, self.kind, self.w = cfg, kind, weights
        self.L = lib(kind)
        self.dt = np_dtype(kind)
        ms = cfg.max_seq if max_seq is None else max_seq
        self.ocfg = OCfg(cfg.n_layers, cfg.hidden, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim,
                         cfg.ffn_dim, cfg.vocab, cfg.n_experts, cfg.top_k, int(cfg.qkv_bias),
                         cfg.sliding_window, ms, n_slots, int(cfg.weight_dtype == 1),
                         int(window_by_mask), cfg.rms_eps, cfg.rope_theta, cfg.rope_pairing, cfg.rope_scaling,
                         cfg.rope_orig_ctx, kv_round(cfg), cfg.rope_factor, cfg.rope_low_freq_factor,
                         cfg.rope_high_freq_factor)
        self.n_slots = n_slots
        arr = (OLayer * cfg.n_layers)()
        for i, lw in enumerate(weights["layers"]):
            for f, _ in OLayer._fields_:
                t = lw.get(f)
                setattr(arr[i], f, _ptr(t) if t is not None else None)
        self._layers = arr
        lm = weights["lm_head"]
        self.h = self.L.create(ctypes.byref(self.ocfg), _ptr(weights["embed"]),
                               _ptr(weights["out_norm"]), _ptr(lm) if lm is not None else None, arr)
        if not self.h:
            raise OracleError("create failed")

    def __del__(self):
        if getattr(self, "h", None):
            self.L.destroy(self.h)
            self.h = None

    def reset(self, slot: int = -1):
        rc = self.L.reset(self.h, slot)
        if rc:
            raise OracleError(rc)

    def length(self, slot: int) -> int:
        return self.L.length(self.h, slot)

    def prefill(self, tokens: Sequence[int], start_pos: int = 0, slot: int = 0,
                rows: Optional[Sequence[int]] = None, partial: bool = False,
                capture: bool = False):
        """Returns dict(logits [n_rows, V], and with capture: hidden [(L+1), n, d],
        router [L, n, E], ids [L, n, k])."""
        c = self.cfg
        tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        n = tok.size
        rws = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
        nr = 1 if rws is None else rws.size
        logits = np.empty((nr, c.vocab), dtype=self.dt)
        hid = rl = ids = None
        if capture:
            hid = np.full((c.n_layers + 1, n, c.hidden), np.nan, dtype=self.dt)
            if c.n_experts:
                rl = np.zeros((c.n_layers, n, c.n_experts), dtype=self.dt)
                ids = np.zeros((c.n_layers, n, c.top_k), dtype=np.int32)
        rc = self.L.prefill(self.h, slot, _ptr(tok), n, start_pos, _ptr(rws) if rws is not None else None,
                            nr, int(partial), _ptr(logits), _ptr(hid), _ptr(rl), _ptr(ids))
        if rc:
            raise OracleError(rc)
        return {"logits": logits, "hidden": hid, "router": rl, "ids": ids}

    def decode(self, tokens: Sequence[int], pos: Sequence[int], capture: bool = False):
        c = self.cfg
        tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        ps = np.ascontiguousarray(np.asarray(pos, dtype=np.int32))
        B = tok.size
        logits = np.empty((B, c.vocab), dtype=self.dt)
        hid = rl = ids = None
        if capture:
            hid = np.empty((c.n_layers + 1, B, c.hidden), dtype=self.dt)
            if c.n_experts:
                rl = np.zeros((c.n_layers, B, c.n_experts), dtype=self.dt)
                ids = np.zeros((c.n_layers, B, c.top_k), dtype=np.int32)
        rc = self.L.decode(self.h, B, _ptr(tok), _ptr(ps), _ptr(logits), _ptr(hid), _ptr(rl), _ptr(ids))
        if rc:
            raise OracleError(rc)
        return {"logits": logits, "hidden": hid, "router": rl, "ids": ids}

    def kv_row(self, layer: int, slot: int, which: int, pos: int):
        out = np.empty(self.cfg.kv_dim, dtype=self.dt)
        self.L.kv_row(self.h, layer, slot, which, pos, _ptr(out))
        return out

    def argmax(self, logits_row) -> int:
        a = np.ascontiguousarray(logits_row, dtype=self.dt)
        return self.L.argmax(_ptr(a), a.size)
