"""Seeded synthetic inputs shared by the HIP path, the CPU oracle and the bench.

This module draws numbers; it holds none of the forward's arithmetic.

Generator (counter-based, so any element can be drawn alone and the result does
not depend on chunking, device or thread order):
  * SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
    generators", OOPSLA 2014): state_i = key + i*gamma, out_i = mix(state_i),
    with gamma = 0x9E3779B97F4A7C15 and the mix64 finalizer below.
  * key(seed, tensor) = out_{tensor+1} of SplitMix64 started at `seed`.
  * element e draws u1 = out_{2e+1}, u2 = out_{2e+2} of SplitMix64 started at
    `key`; u = ((r >> 11) + 0.5) * 2^-53 lies in (0, 1).
  * normal = sqrt(-2 ln u1) * cos(2 pi u2)  (Box & Muller 1958), in float64.
  * a weight is std*normal rounded to fp32, then (matrices) to bf16, RNE.
  * a token id is (out_{i+1} >> 1) mod vocab for stream `tensor`.

torch int64 arithmetic wraps modulo 2^64, which is what SplitMix64 needs; the
right shifts are made logical by masking.  The same code runs on CPU and GPU.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional

import torch

from .configs import ModelConfig, WEIGHT_F32

MASK64 = (1 << 64) - 1
GAMMA_U = 0x9E3779B97F4A7C15
M1_U = 0xBF58476D1CE4E5B9
M2_U = 0x94D049BB133111EB


def _s64(x: int) -> int:
    x &= MASK64
    return x - (1 << 64) if x >= (1 << 63) else x


GAMMA = _s64(GAMMA_U)
M1 = _s64(M1_U)
M2 = _s64(M2_U)


def mix64_int(z: int) -> int:
    """SplitMix64 finalizer on a Python int (exact, unsigned)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * M1_U) & MASK64
    z = ((z ^ (z >> 27)) * M2_U) & MASK64
    return z ^ (z >> 31)


def splitmix64_int(seed: int, i: int) -> int:
    """i-th output (i >= 1) of SplitMix64 started at state `seed`."""
    return mix64_int(seed + i * GAMMA_U)


def _srl(z: torch.Tensor, s: int) -> torch.Tensor:
    return (z >> s) & ((1 << (64 - s)) - 1)


def _mix64(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _srl(z, 30)) * M1
    z = (z ^ _srl(z, 27)) * M2
    return z ^ _srl(z, 31)


def _mix64_(z: torch.Tensor, t: torch.Tensor) -> torch.Tensor:
    """In-place mix64 of z (t is scratch of the same shape); avoids the page
    faults of fresh temporaries, which dominate on the CPU."""
    for s, m in ((30, M1), (27, M2)):
        torch.bitwise_right_shift(z, s, out=t)
        t.bitwise_and_((1 << (64 - s)) - 1)
        z.bitwise_xor_(t)
        z.mul_(m)
    torch.bitwise_right_shift(z, 31, out=t)
    t.bitwise_and_((1 << 33) - 1)
    return z.bitwise_xor_(t)


def tensor_key(seed: int, tensor_id: int) -> int:
    return splitmix64_int(seed, tensor_id + 1)


def _raw(key: int, first: int, count: int, device) -> torch.Tensor:
    """Outputs first+1 .. first+count of SplitMix64 started at `key` (int64)."""
    idx = torch.arange(first + 1, first + count + 1, dtype=torch.int64, device=device)
    return _mix64(idx * GAMMA + _s64(key))


def _uniform_(r: torch.Tensor, t: torch.Tensor, out: torch.Tensor) -> torch.Tensor:
    torch.bitwise_right_shift(r, 11, out=t)
    t.bitwise_and_((1 << 53) - 1)
    out.copy_(t)
    return out.add_(0.5).mul_(2.0 ** -53)


class _Scratch:
    def __init__(self, count: int, device):
        self.idx = torch.empty(count, dtype=torch.int64, device=device)
        self.z = torch.empty_like(self.idx)
        self.t = torch.empty_like(self.idx)
        self.u1 = torch.empty(count, dtype=torch.float64, device=device)
        self.u2 = torch.empty_like(self.u1)


def _normal_into(sc: _Scratch, key: int, start: int, count: int) -> torch.Tensor:
    idx, z, t = sc.idx[:count], sc.z[:count], sc.t[:count]
    u1, u2 = sc.u1[:count], sc.u2[:count]
    torch.arange(start, start + count, dtype=torch.int64, out=idx)
    # u1 from output 2e+1, u2 from output 2e+2 of SplitMix64 started at key
    torch.mul(idx, _s64(2 * GAMMA_U), out=z)
    z.add_(_s64(key + GAMMA_U))
    _uniform_(_mix64_(z, t), t, u1)
    torch.mul(idx, _s64(2 * GAMMA_U), out=z)
    z.add_(_s64(key + 2 * GAMMA_U))
    _uniform_(_mix64_(z, t), t, u2)
    u1.log_().mul_(-2.0).sqrt_()
    u2.mul_(2.0 * math.pi).cos_()
    return u1.mul_(u2)


def normal(seed: int, tensor_id: int, start: int, count: int, device="cpu") -> torch.Tensor:
    """Standard normals of elements [start, start+count) of a tensor, float64."""
    sc = _Scratch(count, device)
    return _normal_into(sc, tensor_key(seed, tensor_id), start, count).clone()


def fill_normal(out: torch.Tensor, seed: int, tensor_id: int, std: float, mean: float = 0.0,
                chunk: int = 1 << 22) -> torch.Tensor:
    """Fill `out` (any float dtype, contiguous) with mean + std*N(0,1), rounded to
    fp32 first and then to out's dtype (round to nearest even)."""
    flat = out.view(-1)
    n = flat.numel()
    chunk = min(chunk, max(n, 1))
    sc = _Scratch(chunk, out.device)
    f32 = torch.empty(chunk, dtype=torch.float32, device=out.device)
    key = tensor_key(seed, tensor_id)
    for s in range(0, n, chunk):
        c = min(chunk, n - s)
        z = _normal_into(sc, key, s, c)
        z.mul_(std).add_(mean)
        f32[:c].copy_(z)
        flat[s:s + c].copy_(f32[:c])
    return out


def tokens(seed: int, stream: int, n: int, vocab: int, device="cpu") -> torch.Tensor:
    """n token ids uniform in [0, vocab) from stream `stream` (int32)."""
    r = _raw(tensor_key(seed, stream), 0, n, device)
    return (_srl(r, 1) % vocab).to(torch.int32)


# Stream ids: prompts of row b, teacher-forced decode tokens of row b.
PROMPT_STREAM = 1_000_000
TEACHER_STREAM = 2_000_000

ROLES = ["attn_norm", "wq", "wk", "wv", "bq", "bk", "bv", "wo", "ffn_norm",
         "w_gate", "w_up", "w_down", "router"]


def tensor_id(layer: int, role: str) -> int:
    if layer < 0:
        return {"embed": 1, "out_norm": 2, "lm_head": 3}[role]
    return 1000 + 16 * layer + ROLES.index(role)


def layer_shapes(cfg: ModelConfig) -> Dict[str, tuple]:
    d, q, kv, f, e = cfg.hidden, cfg.q_dim, cfg.kv_dim, cfg.ffn_dim, cfg.n_experts
    sh = {"attn_norm": (d,), "wq": (q, d), "wk": (kv, d), "wv": (kv, d), "wo": (d, q),
          "ffn_norm": (d,)}
    if cfg.qkv_bias:
        sh.update(bq=(q,), bk=(kv,), bv=(kv,))
    if e:
        sh.update(w_gate=(e, f, d), w_up=(e, f, d), w_down=(e, d, f), router=(e, d))
    else:
        sh.update(w_gate=(f, d), w_up=(f, d), w_down=(d, f))
    return sh


VECTOR_ROLES = ("attn_norm", "ffn_norm", "bq", "bk", "bv", "out_norm")


def make_weights(cfg: ModelConfig, seed: int = 0, device="cpu",
                 layers: Optional[List[int]] = None) -> dict:
    """Random-init weights of a model: matrices N(0, 0.02) in bf16 (fp32 for a
    WEIGHT_F32 model), norm gains 1 + N(0, 0.1) and biases N(0, 0.02) in fp32.

    Returns {"embed", "out_norm", "lm_head" (None when tied), "layers": [dict]}.
    `layers` picks which layer indices to draw (default: all); a model is then
    built from those tensors in that order."""
    mat_dtype = torch.float32 if cfg.weight_dtype == WEIGHT_F32 else torch.bfloat16
    chunk = (1 << 26) if torch.device(device).type == "cuda" else (1 << 22)

    def mat(shape, tid):
        t = torch.empty(shape, dtype=mat_dtype, device=device)
        return fill_normal(t, seed, tid, 0.02, chunk=chunk)

    def vec(shape, tid, mean, std):
        t = torch.empty(shape, dtype=torch.float32, device=device)
        return fill_normal(t, seed, tid, std, mean=mean, chunk=chunk)

    w = {"embed": mat((cfg.vocab, cfg.hidden), tensor_id(-1, "embed")),
         "out_norm": vec((cfg.hidden,), tensor_id(-1, "out_norm"), 1.0, 0.1)}
    w["lm_head"] = None if cfg.tied_embedding else mat((cfg.vocab, cfg.hidden),
                                                       tensor_id(-1, "lm_head"))
    idx = list(range(cfg.n_layers)) if layers is None else list(layers)
    w["layers"] = []
    for l in idx:
        lw = {}
        for role, shape in layer_shapes(cfg).items():
            tid = tensor_id(l, role)
            if role in ("attn_norm", "ffn_norm"):
                lw[role] = vec(shape, tid, 1.0, 0.1)
            elif role in ("bq", "bk", "bv"):
                lw[role] = vec(shape, tid, 0.0, 0.02)
            else:
                lw[role] = mat(shape, tid)
        w["layers"].append(lw)
    return w


def prompts(cfg: ModelConfig, rows: int, length: int, seed: int = 0, device="cpu",
            stream: int = PROMPT_STREAM) -> torch.Tensor:
    """[rows, length] int32 prompt ids; row b uses stream `stream + b`."""
    return torch.stack([tokens(seed, stream + b, length, cfg.vocab, device)
                        for b in range(rows)])
