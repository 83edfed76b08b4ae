"""Parity of the MFMA decode attention (query groups of more than 4 heads,
head_dim 64 or 128; Pantheon "Llama Forward Pass", section "Grouped Query
Attention"; rml "The decoder", section "Attend": one K/V read per group).

Small models with 5 to 8 heads per kv head decode rows of different
lengths together, so a launch holds rows whose last 16-position step is
ragged, rows shorter than one step per wave, and several splits merged by the
split-merge pass.  Every row's logits and every layer's hidden state are
compared with the oracle, with an fp32 and a bf16 K/V cache.
"""
import numpy as np
import pytest
import torch

from decoder_only_forward_amd import configs, synth
from parity_util import Pair, check_argmax, check_hidden, check_logits

pytestmark = pytest.mark.gpu

BASE = configs.TINY_BF16.replace(hidden=128, head_dim=64, ffn_dim=192, max_seq=400)
CASES = [
    BASE.replace(name="g8-hd64", n_heads=8, n_kv_heads=1),
    BASE.replace(name="g5-hd64", n_heads=10, n_kv_heads=2),
    BASE.replace(name="g6-hd64", n_heads=12, n_kv_heads=2),
    BASE.replace(name="g8-hd64-kvbf16", n_heads=8, n_kv_heads=1, kv_bf16=True),
    BASE.replace(name="g7-hd128", n_heads=14, n_kv_heads=2, head_dim=128, hidden=256),
]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_mfma_decode_rows_of_different_lengths(cfg):
    print(f"[decode mfma] {cfg.name}", flush=True)
    lens = [300, 37, 5, 130]
    B = len(lens)
    pair = Pair(cfg, n_slots=B, max_prefill=max(lens))
    prompts = [synth.tokens(0, synth.PROMPT_STREAM + b, n, cfg.vocab).tolist() for b, n in enumerate(lens)]
    nxt = []
    for b in range(B):
        pair.gpu.prefill(prompts[b], seq=b)
        r = pair.ora.prefill(prompts[b], slot=b)
        nxt.append(int(np.argmax(r["logits"][0])))
    for s in range(3):
        pos = [n + s for n in lens]
        hid, _, _ = pair.capture_buffers(B)
        g = pair.gpu.decode(nxt, pos).cpu().numpy()
        r = pair.ora.decode(nxt, pos, capture=True)
        for b in range(B):
            check_logits(g[b], r["logits"][b], f"{cfg.name} row {b} step {s}", **pair.tol)
            check_argmax(g[b], r["logits"][b], f"{cfg.name} row {b} step {s}", **pair.tol)
        check_hidden(hid.cpu().numpy(), r["hidden"], f"{cfg.name} step {s}", **pair.tol)
        nxt = [int(np.argmax(r["logits"][b])) for b in range(B)]
    # a second batch shape: one row alone (many splits of few positions)
    g1 = pair.gpu.decode([nxt[0]], [lens[0] + 3]).cpu().numpy()[0]
    r1 = pair.ora.decode([nxt[0]], [lens[0] + 3])["logits"][0]
    check_logits(g1, r1, f"{cfg.name} B=1", **pair.tol)
