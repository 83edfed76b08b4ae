"""dec_create_noalloc: a handle whose workspace is the library's own device
array gives the results of a dec_create handle on the same weights.

Each test makes one handle of each kind over the same device weights and
runs the same calls on both: a prefill and batched decode steps, then, after a
reset, a smaller prefill and decode (two calls in a row, the second smaller).
Results must be identical (same kernels, same launch shapes) and within the
parity tolerances of the oracle.  A second live handle on the device is
refused, and the array serves a new handle once the first is destroyed.
"""
import numpy as np
import pytest
import torch

from decoder_only_forward_amd import configs, synth
from decoder_only_forward_amd import dec as D
from oracle import oracle as O
from parity_util import check_argmax, check_logits, to_device

pytestmark = pytest.mark.gpu


def _pair_calls(cfg, B, P_big, P_small, steps):
    print(f"[noalloc] {cfg.name} B={B} P={P_big}/{P_small}", flush=True)
    w = synth.make_weights(cfg)
    wd = to_device(w)
    ref = D.DecModel(cfg, wd, max_batch=B, max_prefill=P_big)
    na = D.DecModel(cfg, wd, max_batch=B, max_prefill=P_big, noalloc=True)
    assert na.workspace is None
    ora = O.OracleModel(cfg, w, n_slots=B)
    for P in (P_big, P_small):
        for m in (ref, na):
            m.reset()
        ora.reset()
        pr = synth.prompts(cfg, B, P)
        outs = []
        for m in (ref, na):
            pre = [m.prefill(pr[b].tolist(), seq=b).cpu().numpy() for b in range(B)]
            toks = [int(np.argmax(p)) for p in pre]
            dec = []
            for s in range(steps):
                lg = m.decode(toks, [P + s] * B).cpu().numpy()
                dec.append(lg)
                toks = [int(np.argmax(lg[b])) for b in range(B)]
            outs.append((pre, dec))
        for b in range(B):
            assert np.array_equal(outs[0][0][b], outs[1][0][b]), f"P={P} prefill row {b}"
        for s in range(steps):
            assert np.array_equal(outs[0][1][s], outs[1][1][s]), f"P={P} decode step {s}"
        # and the oracle, on the noalloc handle's results
        pre, dec = outs[1]
        toks = []
        for b in range(B):
            r = ora.prefill(pr[b].tolist(), slot=b)["logits"][0]
            check_logits(pre[b], r, f"noalloc P={P} prefill row {b}")
            check_argmax(pre[b], r, f"noalloc P={P} prefill row {b}")
            toks.append(int(np.argmax(pre[b])))
        for s in range(steps):
            r = ora.decode(toks, [P + s] * B)["logits"]
            for b in range(B):
                check_logits(dec[s][b], r[b], f"noalloc P={P} step {s} row {b}")
            toks = [int(np.argmax(dec[s][b])) for b in range(B)]
    # one live noalloc handle per device
    with pytest.raises(D.DecError) as e:
        D.DecModel(cfg, wd, max_batch=1, max_prefill=8, noalloc=True)
    assert e.value.code == D.DEC_ERR_INVALID
    na.close()
    ref.close()


def test_noalloc_handle_equals_workspace_handle_tiny():
    _pair_calls(configs.TINY_BF16, B=2, P_big=12, P_small=5, steps=3)


def test_noalloc_handle_equals_workspace_handle_smollm2():
    """SmolLM2-135M at 4 slots and 128-token prefills (60 MiB of the 64 MiB
    array), then 20-token prefills; decode steps replay captured graphs."""
    _pair_calls(configs.SMOLLM2, B=4, P_big=128, P_small=20, steps=3)


def test_noalloc_array_serves_the_next_handle_and_refuses_oversize():
    cfg = configs.TINY_MOE
    w = synth.make_weights(cfg)
    wd = to_device(w)
    a = D.DecModel(cfg, wd, max_batch=1, max_prefill=8, noalloc=True)
    toks = synth.tokens(0, synth.PROMPT_STREAM, 8, cfg.vocab).tolist()
    la = a.prefill(toks).cpu().numpy()
    a.close()
    b = D.DecModel(cfg, wd, max_batch=1, max_prefill=8, noalloc=True)
    lb = b.prefill(toks).cpu().numpy()
    b.close()
    assert np.array_equal(la, lb)
    with pytest.raises(D.DecError) as e:
        D.DecModel(configs.SMOLLM2, to_device(synth.make_weights(configs.SMOLLM2)), max_batch=32,
                   max_prefill=128, noalloc=True)
    assert e.value.code == D.DEC_ERR_NOMEM
