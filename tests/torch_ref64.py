"""An independent float64 forward of the decoder, built from torch library
routines, used only to pin the CPU oracle's composition of the layer.

It shares nothing with oracle/oracle.c: projections are `F.linear` on the
[out][in] weight matrices, RMSNorm is `F.rms_norm`, attention is
`F.scaled_dot_product_attention` with `enable_gqa` and an explicit boolean mask
over a plain (linear, never circular) list of keys, RoPE multiplies complex
numbers by unit phasors from `torch.polar`, MoE routing takes a stable
descending sort of the softmax.  It works on whole sequences: position p's
result is row p of one causal pass over tokens 0..p (the rule that single-pass
prefill equals per-token forward calls, sipllm "Transformer forward pass",
section "Single-pass prefill").

What it computes (Pantheon "Llama Forward Pass", sections "Forward Pass Flow",
"RMSNorm", "RoPE", "Grouped Query Attention", "SwiGLU FFN", "Mixture of Experts
(Mixtral)", "Sliding Window (Mistral)"; rml "The decoder", sections "Rotary
embeddings", "Attend", "Mixture of experts", "One forward pass"):

    x = E[tok]
    per layer: a = rmsnorm(x, attn_norm); q, k, v = Wq a + bq, Wk a + bk, Wv a + bv
               rotate pairs of q and k by pos * f_i; (optionally round k, v to bf16)
               o = softmax(q k^T / sqrt(hd), causal [window] mask) v, head h -> kv head h*n_kv/n_heads
               x += Wo o; b = rmsnorm(x, ffn_norm)
               x += Wd (silu(Wg b) * Wu b)     or     the top-k renormalised expert mixture
    logits = W_out rmsnorm(x, out_norm)
"""
from __future__ import annotations

import math

import torch
import torch.nn.functional as F

D = torch.float64


def _w(t):
    return None if t is None else t.to(D)


def inv_freq(cfg) -> torch.Tensor:
    """Frequency of pair i: theta^(-2i/hd); with llama3 scaling, pairs whose
    wavelength 2 pi / f exceeds orig_ctx / low turn `factor` times slower,
    those under orig_ctx / high keep f, and the band between blends linearly in
    orig_ctx / wavelength (rml "The decoder", "Rotary embeddings")."""
    hd = cfg.head_dim
    f = cfg.rope_theta ** (-torch.arange(0, hd, 2, dtype=D) / hd)
    if cfg.rope_scaling == 1:
        wl = 2 * math.pi / f
        lo_wl = cfg.rope_orig_ctx / cfg.rope_low_freq_factor
        hi_wl = cfg.rope_orig_ctx / cfg.rope_high_freq_factor
        s = (cfg.rope_orig_ctx / wl - cfg.rope_low_freq_factor) / (
            cfg.rope_high_freq_factor - cfg.rope_low_freq_factor)
        mid = (1 - s) * f / cfg.rope_factor + s * f
        f = torch.where(wl < hi_wl, f, torch.where(wl > lo_wl, f / cfg.rope_factor, mid))
    return f


def rope(h: torch.Tensor, pos: torch.Tensor, cfg) -> torch.Tensor:
    """h [n, heads, hd] at positions pos [n]: each pair (a, b) read as the complex
    number a + ib and multiplied by exp(i pos f_pair).  Adjacent pairing takes
    (2i, 2i+1), halves pairing (i, i + hd/2)."""
    n, nh, hd = h.shape
    ang = pos.to(D)[:, None] * inv_freq(cfg)[None, :]                      # [n, hd/2]
    ph = torch.polar(torch.ones_like(ang), ang)[:, None, :]                # [n, 1, hd/2]
    if cfg.rope_pairing == 0:
        z = torch.view_as_complex(h.reshape(n, nh, hd // 2, 2).contiguous()) * ph
        return torch.view_as_real(z).reshape(n, nh, hd)
    z = torch.complex(h[..., : hd // 2], h[..., hd // 2:]) * ph
    return torch.cat([z.real, z.imag], dim=-1)


def _bf16(t):
    return t.to(torch.float32).to(torch.bfloat16).to(D)


def _sig16(t):
    """The fp32 value of t rounded to 16 significant bits, ties to even
    (frexp's mantissa in [0.5, 1) scaled by 2^16 and rounded half to even)."""
    m, e = torch.frexp(t.to(torch.float32).to(torch.float64))
    return torch.ldexp(torch.round(m * 65536.0), e - 16)


def route(r: torch.Tensor, k: int):
    """Router logits r [E] -> (ids [k], weights [k]): softmax, the k largest
    probabilities with ties to the lower id (a stable descending sort keeps
    equal values in id order), divided by their sum."""
    p = torch.softmax(r, dim=-1)
    order = torch.sort(p, descending=True, stable=True).indices[:k]
    sel = p[order]
    return order, sel / sel.sum()


def forward(cfg, w: dict, tokens) -> dict:
    """Causal forward of one sequence at positions 0..n-1.  Returns
    hidden [(L+1), n, d] (after the embedding and each layer), logits [n, V],
    router [L, n, E] and ids [L, n, k] (MoE)."""
    tok = torch.as_tensor(list(tokens), dtype=torch.long)
    n = tok.numel()
    d, hd, nh, nkv = cfg.hidden, cfg.head_dim, cfg.n_heads, cfg.n_kv_heads
    pos = torch.arange(n)
    i = pos[:, None]
    j = pos[None, :]
    mask = j <= i
    if cfg.sliding_window:
        mask = mask & (j > i - cfg.sliding_window)
    x = _w(w["embed"])[tok]
    hidden = [x.clone()]
    routers, ids_all = [], []
    for L in w["layers"]:
        a = F.rms_norm(x, (d,), weight=_w(L["attn_norm"]), eps=cfg.rms_eps)
        q = F.linear(a, _w(L["wq"]), _w(L.get("bq")))
        k = F.linear(a, _w(L["wk"]), _w(L.get("bk")))
        v = F.linear(a, _w(L["wv"]), _w(L.get("bv")))
        q = rope(q.view(n, nh, hd), pos, cfg)
        k = rope(k.view(n, nkv, hd), pos, cfg)
        v = v.view(n, nkv, hd)
        if cfg.kv_bf16:
            k, v = _bf16(k), _bf16(v)
        if getattr(cfg, "kv_f24", False):
            k, v = _sig16(k), _sig16(v)
        o = F.scaled_dot_product_attention(q.transpose(0, 1)[None], k.transpose(0, 1)[None],
                                           v.transpose(0, 1)[None], attn_mask=mask, enable_gqa=True)
        o = o[0].transpose(0, 1).reshape(n, nh * hd)
        x = x + F.linear(o, _w(L["wo"]))
        b = F.rms_norm(x, (d,), weight=_w(L["ffn_norm"]), eps=cfg.rms_eps)
        if not cfg.n_experts:
            y = F.linear(F.silu(F.linear(b, _w(L["w_gate"]))) * F.linear(b, _w(L["w_up"])), _w(L["w_down"]))
        else:
            r = F.linear(b, _w(L["router"]))
            routers.append(r)
            y = torch.zeros_like(x)
            ids_l = []
            for t in range(n):
                ids, wt = route(r[t], cfg.top_k)
                ids_l.append(ids)
                for e, we in zip(ids.tolist(), wt):
                    g = F.linear(b[t], _w(L["w_gate"][e]))
                    u = F.linear(b[t], _w(L["w_up"][e]))
                    y[t] += we * F.linear(F.silu(g) * u, _w(L["w_down"][e]))
            ids_all.append(torch.stack(ids_l))
        x = x + y
        hidden.append(x.clone())
    head = w["embed"] if cfg.tied_embedding or w.get("lm_head") is None else w["lm_head"]
    logits = F.linear(F.rms_norm(x, (d,), weight=_w(w["out_norm"]), eps=cfg.rms_eps), _w(head))
    out = {"hidden": torch.stack(hidden).numpy(), "logits": logits.numpy()}
    if cfg.n_experts:
        out["router"] = torch.stack(routers).numpy()
        out["ids"] = torch.stack(ids_all).numpy()
    return out
