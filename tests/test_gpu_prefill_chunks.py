"""Parity of the prefill attention when its row blocks are split into key
chunks (Pantheon "Llama Forward Pass", section "Flash (Blocked) Prefill
Attention"; rml "The decoder", section "Attend": the online softmax's state of
disjoint key ranges combines exactly).

A model with the Qwen2.5-0.5B attention shape (14 query heads on 2 kv heads,
head_dim 64) prefills 700 tokens: 20 row blocks of 36 rows x 2 kv heads is far
fewer blocks than the CUs, so every row block's key tiles are cut into chunks of
2 tiles and merged, the last row block's into 6.  An append of 200 tokens from
position 700 splits again, with chunks that start inside the history.  Every
row's logits and every layer's hidden state are compared with the oracle, with
an fp32 and a bf16 K/V cache.
"""
import numpy as np
import pytest

from decoder_only_forward_amd import configs, synth
from parity_util import Pair, check_argmax, check_hidden, check_logits

pytestmark = pytest.mark.gpu

BASE = configs.QWEN25.replace(name="qwen-attn-2l", n_layers=2, ffn_dim=1024, vocab=512, tied_embedding=False,
                              max_seq=1024)


@pytest.mark.parametrize("cfg", [BASE, BASE.replace(name="qwen-attn-2l-kvbf16", kv_bf16=True)],
                         ids=lambda c: c.name)
def test_prefill_attention_in_key_chunks(cfg):
    print(f"[prefill chunks] {cfg.name}", flush=True)
    P, A = 700, 200
    pair = Pair(cfg, max_prefill=P, max_seq=cfg.max_seq)
    toks = synth.tokens(0, synth.PROMPT_STREAM, P + A, cfg.vocab).tolist()
    for start, n in ((0, P), (P, A)):
        what = f"{cfg.name} rows {start}..{start + n - 1}"
        hid, _, _ = pair.capture_buffers(n)
        g = pair.gpu.prefill(toks[start:start + n], start_pos=start, all_logits=True).cpu().numpy()
        r = pair.ora.prefill(toks[start:start + n], start_pos=start, rows=list(range(n)), capture=True)
        for t in range(n):
            check_logits(g[t], r["logits"][t], f"{what}: row {t}", **pair.tol)
            check_argmax(g[t], r["logits"][t], f"{what}: row {t}", **pair.tol)
        check_hidden(hid.cpu().numpy(), r["hidden"], what, **pair.tol)
    # then a decode step reads the whole history
    nxt = int(np.argmax(r["logits"][-1]))
    g = pair.gpu.decode([nxt], [P + A]).cpu().numpy()[0]
    rd = pair.ora.decode([nxt], [P + A])["logits"][0]
    check_logits(g, rd, f"{cfg.name} decode after the append", **pair.tol)
