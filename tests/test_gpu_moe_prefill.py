"""Parity of the MoE prefill path (more than 64 rows): router logits and top-k
formed per token in one kernel, the stable grouping by expert, the grouped
MFMA GEMM (512-feature x 128-row tiles per expert) with silu(gate) * up in the
gate|up epilogue and the down projection split over k.

Edge cases: experts holding more than one 128-row tile with a ragged last
32-row sub-tile (4 experts, top-2, 300 tokens: ~150 rows each), experts with
no rows at all (32 experts, top-1, 100 tokens), feature counts below one tile
(tiny widths), and a long inner dimension (a SmolLM2-width MoE).  Every row's
logits, every layer's hidden state and every expert choice are compared with
the oracle (Pantheon "Llama Forward Pass", section "Mixture of Experts
(Mixtral)"; zLLM "The Algorithm Layer", section 4, grouped expert execution).
"""
import numpy as np
import pytest
import torch

from decoder_only_forward_amd import configs, synth
from parity_util import Pair, check_argmax, check_experts, check_hidden, check_logits

pytestmark = pytest.mark.gpu


def _prefill_all(cfg, T, then_decode=2):
    print(f"[moe prefill] {cfg.name} T={T}", flush=True)
    pair = Pair(cfg, max_prefill=T, max_seq=T + then_decode + 1)
    prompt = synth.tokens(0, synth.PROMPT_STREAM, T, cfg.vocab).tolist()
    hid, ids, rl = pair.capture_buffers(T)
    g = pair.gpu.prefill(prompt, all_logits=True).cpu().numpy()
    r = pair.ora.prefill(prompt, rows=list(range(T)), capture=True)
    torch.cuda.synchronize()
    for t in range(T):
        check_logits(g[t], r["logits"][t], f"{cfg.name} row {t}")
        check_argmax(g[t], r["logits"][t], f"{cfg.name} row {t}")
    check_hidden(hid.cpu().numpy(), r["hidden"], f"{cfg.name} prefill")
    gi = ids.cpu().numpy()
    check_experts(gi, r["ids"], r["router"], cfg.top_k, f"{cfg.name} prefill")
    counts = np.stack([np.bincount(r["ids"][l].reshape(-1), minlength=cfg.n_experts) for l in range(cfg.n_layers)])
    nxt = int(np.argmax(r["logits"][-1]))
    for s in range(then_decode):
        g = pair.gpu.decode([nxt], [T + s]).cpu().numpy()[0]
        rd = pair.ora.decode([nxt], [T + s])["logits"][0]
        check_logits(g, rd, f"{cfg.name} decode {s}")
        nxt = int(np.argmax(rd))
    return counts


def test_moe_prefill_experts_with_two_row_tiles():
    cfg = configs.TINY_BF16.replace(name="tiny-bf16-moe4", n_experts=4, top_k=2)
    counts = _prefill_all(cfg, 300)
    assert counts.max() > 128 and (counts % 32 != 0).any()   # two row tiles, a ragged sub-tile


def test_moe_prefill_experts_without_rows():
    cfg = configs.TINY_BF16.replace(name="tiny-bf16-moe32-top1", n_experts=32, top_k=1)
    counts = _prefill_all(cfg, 100)
    assert (counts == 0).any()                                 # some expert of some layer has no rows


def test_moe_prefill_smollm2_width():
    """576-wide tokens, ffn 1536 per expert, 8 experts top-2, 2 layers, 160 tokens."""
    cfg = configs.SMOLLM2.replace(name="smollm2-moe-2l", n_layers=2, n_experts=8, top_k=2, vocab=4096,
                                  tied_embedding=False)
    _prefill_all(cfg, 160)
