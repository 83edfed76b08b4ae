"""Every K/V cache row against the oracle's after prefills and one batched
decode step: the decode attention kernel stores each row's new rotated key
and value in its prologue, at slot pos % max_seq of a ring (Pantheon "Llama
Forward Pass", "Sliding Window (Mistral)") or at pos, and the rows the
prefills wrote must stay as they were.  Cache layout [layer][slot][kv head]
[max_seq][head_dim] at the start of the workspace, K then V (256-byte aligned);
fp32, nearest-even bf16 bits, or 24-bit rows (head_dim upper halves, then
head_dim third bytes in blocks of 8)."""
import numpy as np
import pytest
import torch

from decoder_only_forward_amd import configs, synth
from parity_util import Pair, rel_l2, tol

pytestmark = pytest.mark.gpu

CASES = [configs.TINY_WINDOW, configs.TINY_WINDOW.replace(name="tiny-window-kvbf16", kv_bf16=True),
         configs.TINY_WINDOW.replace(name="tiny-window-kvf24", kv_f24=True),
         configs.TINY_BF16, configs.TINY_KVBF16, configs.TINY_KVF24]


def _caches(pair):
    c, g = pair.cfg, pair.gpu
    S, ms = g.ccfg.max_batch, g.ccfg.max_seq
    es = 2 if c.kv_bf16 else (3 if c.kv_f24 else 4)
    hd = c.head_dim
    n = c.n_layers * S * c.n_kv_heads * ms * hd
    kbytes = n * es
    voff = (kbytes + 255) // 256 * 256
    raw = g.workspace[: voff + kbytes].cpu().numpy()
    out = []
    for off in (0, voff):
        b = raw[off: off + kbytes]
        if es == 2:
            a = (np.frombuffer(b.tobytes(), dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
        elif es == 3:
            rows = np.frombuffer(b.tobytes(), dtype=np.uint8).reshape(-1, 3 * hd)
            hi = rows[:, : 2 * hd].copy().view(np.uint16).astype(np.uint32)
            # third bytes by blocks of 8 elements, block j at 16 (j % L) + 8 (j // L), L = hd / 16
            L = hd // 16
            e = np.arange(hd)
            lo = rows[:, 2 * hd + 16 * ((e // 8) % L) + 8 * ((e // 8) // L) + e % 8].astype(np.uint32)
            a = ((hi << 16) | (lo << 8)).view(np.float32)
        else:
            a = np.frombuffer(b.tobytes(), dtype=np.float32)
        out.append(a.reshape(c.n_layers, S, c.n_kv_heads, ms, hd))
    return out, ms


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_decode_stores_each_rows_new_kv_row_at_its_slot(cfg):
    pair = Pair(cfg, n_slots=3, max_prefill=16)
    lens = [3, 5, 7]          # with a 5-slot ring, 7 positions have wrapped
    for b, n in enumerate(lens):
        toks = synth.tokens(b, synth.PROMPT_STREAM, n, cfg.vocab).tolist()
        pair.gpu.prefill(toks, seq=b)
        pair.ora.prefill(toks, slot=b)
    nxt = [11, 22, 33]
    pair.gpu.decode(nxt, lens)
    pair.ora.decode(nxt, lens)
    torch.cuda.synchronize()
    (kc, vc), ms = _caches(pair)
    ring = cfg.sliding_window > 0 and ms == cfg.sliding_window
    bound = tol(cfg)["rel"]
    for b, n in enumerate(lens):
        for p in range(max(0, n + 1 - ms), n + 1):      # the readable positions, the new one last
            s = p % ms if ring else p
            for which, cache in ((0, kc), (1, vc)):
                for layer in range(cfg.n_layers):
                    got = cache[layer, b, :, s, :].reshape(-1)
                    ref = pair.ora.kv_row(layer, b, which, p)
                    r = rel_l2(got, ref)
                    assert r <= bound, f"{cfg.name} slot {b} position {p} {'kv'[which]} layer {layer}: rel L2 {r:.2e}"
    pair.gpu.close()
