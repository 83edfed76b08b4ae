"""The C ABI boundary on the host (no GPU): the library loads, exports every
function include/dec.h declares, and rejects bad calls before touching the
device, leaving every KV length unchanged (rml "The decoder", section "One
forward pass", step 1)."""
import ctypes
import os
import re

import numpy as np
import pytest

from decoder_only_forward_amd import configs
from decoder_only_forward_amd import dec as D

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    if not os.path.exists(D.LIB_PATH):
        pytest.skip("libdec.so not built (run __graft_entry__.build())")
    return D.load()


def test_header_exports_are_all_present():
    L = _lib()
    with open(os.path.join(ROOT, "include", "dec.h")) as f:
        names = re.findall(r"DEC_API\s+[\w\s\*]*?\b(dec_\w+)\s*\(", f.read())
    assert len(names) >= 14 and set(D.EXPORTS) <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_probe_header_exports_are_all_present():
    from decoder_only_forward_amd import probe
    if not os.path.exists(probe.LIB_PATH):
        pytest.skip("libdec_probe.so not built (run __graft_entry__.build())")
    L = probe.load()
    with open(os.path.join(ROOT, "include", "dec_probe.h")) as f:
        names = re.findall(r"\bint\s+(decp_\w+)\s*\(", f.read())
    assert set(names) == set(probe.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_workspace_bytes_is_host_only_and_validates():
    _lib()
    n = D.workspace_bytes(configs.MISTRAL, max_batch=32, max_prefill=4096)
    kv = 2 * 32 * 32 * 8 * 4096 * 128 * 4          # fp32 K and V of 32 slots
    assert n >= kv
    assert D.workspace_bytes(configs.MISTRAL.replace(n_kv_heads=5), 1, 1) == 0     # heads do not split
    assert D.workspace_bytes(configs.TINY.replace(head_dim=15), 1, 1) == 0         # odd head_dim
    assert D.workspace_bytes(configs.TINY, 1, 0) == 0


def test_bf16_cache_halves_the_kv_bytes():
    _lib()
    f32 = D.workspace_bytes(configs.MISTRAL, max_batch=32, max_prefill=4096)
    b16 = D.workspace_bytes(configs.MISTRAL.replace(kv_bf16=True), max_batch=32, max_prefill=4096)
    kv = 2 * 32 * 32 * 8 * 4096 * 128 * 2        # K and V of 32 slots, 2 bytes saved per element
    chunk = 2 * 4096 * 8 * 128 * 2                # the ring's deferred-commit chunk K/V (max_prefill rows)
    # prefill attention's K/V tile images (64 tiles x 8 heads): bf16 (hi, lo) pairs of K and V^T
    # (72 KiB per tile, padded rows) against the bf16 cache's exact halves (40 KiB per tile)
    img = 64 * 8 * (73728 - 40960)
    assert f32 - b16 == kv + chunk + img


def test_f24_cache_takes_three_quarters_of_the_kv_bytes():
    _lib()
    f32 = D.workspace_bytes(configs.MISTRAL, max_batch=32, max_prefill=4096)
    f24 = D.workspace_bytes(configs.MISTRAL.replace(kv_f24=True), max_batch=32, max_prefill=4096)
    kv = 2 * 32 * 32 * 8 * 4096 * 128 * 1        # K and V of 32 slots, 1 byte saved per element
    chunk = 2 * 4096 * 8 * 128 * 1                # the ring's deferred-commit chunk K/V
    assert f32 - f24 == kv + chunk                 # same (hi, lo) tile images as the fp32 cache
    assert D.kv_dtype(configs.MISTRAL.replace(kv_f24=True)) == D.DEC_KV_F24


def _create(cfg, max_batch=2, max_prefill=8, ws=None, ws_bytes=None, layer_field=None, **over):
    L = _lib()
    c = D.make_config(cfg, max_batch, max_prefill)
    for k, v in over.items():
        setattr(c, k, v)
    need = L.dec_workspace_bytes(ctypes.byref(c))
    fake = 0x7F0000000000          # never dereferenced: create only validates and records
    layers = (D.DecLayerWeights * cfg.n_layers)()
    for i in range(cfg.n_layers):
        for f, _ in D.DecLayerWeights._fields_:
            setattr(layers[i], f, fake)
    if layer_field is not None:    # (field, address) set in the last layer
        setattr(layers[cfg.n_layers - 1], *layer_field)
    w = D.DecWeights(ctypes.sizeof(D.DecWeights), fake, fake, fake, layers)
    h = ctypes.c_void_p()
    rc = L.dec_create(ctypes.byref(c), ctypes.byref(w), ws if ws is not None else fake,
                      ws_bytes if ws_bytes is not None else need, None, ctypes.byref(h))
    return rc, h, L


def test_create_validation():
    assert _create(configs.TINY, ws_bytes=16)[0] == D.DEC_ERR_NOMEM
    assert _create(configs.TINY, ws=0x7F0000000001)[0] == D.DEC_ERR_INVALID      # misaligned
    # weights are read in 16-byte words: a pointer off that grid is refused
    assert _create(configs.TINY, layer_field=("wq", 0x7F0000000008))[0] == D.DEC_ERR_INVALID
    assert _create(configs.QWEN25, layer_field=("bk", 0x7F0000000004))[0] == D.DEC_ERR_INVALID
    rc, h, L = _create(configs.TINY, layer_field=("w_down", 0x7F0000000010))
    assert rc == D.DEC_OK
    L.dec_destroy(h)
    assert _create(configs.TINY, struct_size=8)[0] == D.DEC_ERR_INVALID
    assert _create(configs.TINY, head_dim=32)[0] == D.DEC_ERR_UNSUPPORTED
    assert _create(configs.TINY, max_batch=65)[0] == D.DEC_ERR_UNSUPPORTED
    assert _create(configs.TINY, n_experts=2, top_k=3)[0] == D.DEC_ERR_INVALID   # top_k > n_experts
    assert _create(configs.TINY_BF16, ffn_dim=100)[0] == D.DEC_ERR_UNSUPPORTED    # bf16 tiles need 64 | ffn
    assert _create(configs.TINY_WINDOW, max_seq=6)[0] == D.DEC_ERR_INVALID       # ring longer than the window
    assert _create(configs.TINY, kv_dtype=3)[0] == D.DEC_ERR_INVALID              # no such cache type
    for cfg in (configs.TINY_KVBF16, configs.TINY_KVF24):
        rc, h, L = _create(cfg)
        assert rc == D.DEC_OK
        L.dec_destroy(h)
    rc, h, L = _create(configs.TINY)
    assert rc == D.DEC_OK
    L.dec_destroy(h)


def test_bad_calls_change_nothing():
    rc, h, L = _create(configs.TINY, max_batch=2, max_prefill=8)
    assert rc == D.DEC_OK
    fake_logits = ctypes.c_void_p(0x7F0000000000)
    tok = np.array([1, 2, 3], dtype=np.int32)
    bad = np.array([1, configs.TINY.vocab], dtype=np.int32)
    pos = np.array([0, 0], dtype=np.int32)
    cases = [
        (L.dec_prefill, (h, 0, bad.ctypes.data, 2, 0, fake_logits), D.DEC_ERR_INVALID),   # id >= vocab
        (L.dec_prefill, (h, 0, tok.ctypes.data, 0, 0, fake_logits), D.DEC_ERR_INVALID),   # empty
        (L.dec_prefill, (h, 2, tok.ctypes.data, 3, 0, fake_logits), D.DEC_ERR_INVALID),   # no slot 2
        (L.dec_prefill, (h, 0, tok.ctypes.data, 3, 1, fake_logits), D.DEC_ERR_INVALID),   # not the length
        (L.dec_prefill, (h, 0, np.zeros(9, np.int32).ctypes.data, 9, 0, fake_logits), D.DEC_ERR_RANGE),
        (L.dec_decode, (h, 3, tok.ctypes.data, np.zeros(3, np.int32).ctypes.data, fake_logits), D.DEC_ERR_INVALID),
        (L.dec_decode, (h, 2, tok.ctypes.data, np.array([0, 5], np.int32).ctypes.data, fake_logits),
         D.DEC_ERR_INVALID),
        (L.dec_decode, (h, 2, bad.ctypes.data, pos.ctypes.data, fake_logits), D.DEC_ERR_INVALID),
        (L.dec_kv_reset, (h, 5), D.DEC_ERR_INVALID),
        (L.dec_greedy, (h, fake_logits, 3, tok.ctypes.data), D.DEC_ERR_INVALID),
        (L.dec_prefill_ex, (h, 0, tok.ctypes.data, 3, 0, fake_logits, 2), D.DEC_ERR_INVALID),   # all_logits 0/1
        (L.dec_prefill_ex, (h, 0, bad.ctypes.data, 2, 0, fake_logits, 1), D.DEC_ERR_INVALID),
        (L.dec_decode_greedy, (h, 2, tok.ctypes.data, 0, fake_logits, fake_logits), D.DEC_ERR_INVALID),  # 0 steps
        (L.dec_decode_greedy, (h, 3, tok.ctypes.data, 2, fake_logits, fake_logits), D.DEC_ERR_INVALID),  # B > slots
        (L.dec_decode_greedy, (h, 2, bad.ctypes.data, 2, fake_logits, fake_logits), D.DEC_ERR_INVALID),
        (L.dec_decode_greedy, (h, 2, tok.ctypes.data, 17, fake_logits, fake_logits), D.DEC_ERR_RANGE),  # > max_seq
        (L.dec_decode_greedy, (h, 2, tok.ctypes.data, 2, None, fake_logits), D.DEC_ERR_INVALID),
    ]
    for fn, args, want in cases:
        assert fn(*args) == want, (fn.__name__, args)
        assert L.dec_kv_length(h, 0) == 0 and L.dec_kv_length(h, 1) == 0
    assert L.dec_kv_length(h, 2) == D.DEC_ERR_INVALID
    assert L.dec_status_str(D.DEC_ERR_RANGE) == b"out of range"
    L.dec_destroy(h)


def test_capacity_without_window_is_range_error():
    rc, h, L = _create(configs.TINY, max_batch=1, max_prefill=64)     # max_seq 16
    tok = np.zeros(17, dtype=np.int32)
    assert L.dec_prefill(h, 0, tok.ctypes.data, 17, 0, ctypes.c_void_p(0x7F0000000000)) == D.DEC_ERR_RANGE
    assert L.dec_kv_length(h, 0) == 0
    L.dec_destroy(h)


def test_create_noalloc_checks_before_the_device():
    """dec_create_noalloc refuses a workspace larger than its static array, and
    a bad config, on the host before any device call."""
    L = _lib()
    fake = 0x7F0000000000
    for cfg, mb, mp, want in ((configs.MISTRAL, 1, 64, D.DEC_ERR_NOMEM),
                              (configs.SMOLLM2, 32, 128, D.DEC_ERR_NOMEM),
                              (configs.TINY.replace(head_dim=15), 1, 8, D.DEC_ERR_INVALID)):
        c = D.make_config(cfg, mb, mp)
        need = L.dec_workspace_bytes(ctypes.byref(c))
        assert want != D.DEC_ERR_NOMEM or need > D.DEC_NOALLOC_WORKSPACE_BYTES
        layers = (D.DecLayerWeights * cfg.n_layers)()
        for i in range(cfg.n_layers):
            for f, _ in D.DecLayerWeights._fields_:
                setattr(layers[i], f, fake)
        w = D.DecWeights(ctypes.sizeof(D.DecWeights), fake, fake, fake, layers)
        h = ctypes.c_void_p()
        assert L.dec_create_noalloc(ctypes.byref(c), ctypes.byref(w), None, ctypes.byref(h)) == want
        assert not h.value
    c = D.make_config(configs.TINY, 1, 8)
    assert L.dec_create_noalloc(ctypes.byref(c), None, None, None) == D.DEC_ERR_INVALID
    assert D.workspace_bytes(configs.SMOLLM2, 4, 128) <= D.DEC_NOALLOC_WORKSPACE_BYTES


def _f8_matrix_bytes(N, K, silu):
    """Workspace bytes of one matrix converted for fp16 + fp8 prefill operands:
    rows padded to 256-row tiles (a gate|up tile holds 128 features of each),
    the fp16 copy, 256-aligned (the fp8 pass reads its upper bytes)."""
    npad = ((N + 127) // 128) * 256 if silu else ((N + 255) // 256) * 256
    return (npad * K * 2 + 255) // 256 * 256


def test_fp16_fp8_prefill_operands_workspace_and_validation():
    _lib()
    m = configs.MISTRAL
    base = D.workspace_bytes(m, max_batch=32, max_prefill=4096)
    f8 = D.workspace_bytes(m.replace(prefill_fp8=True), max_batch=32, max_prefill=4096)
    d, qd, kvd, F = m.hidden, m.q_dim, m.kv_dim, m.ffn_dim
    per_layer = _f8_matrix_bytes(qd + 2 * kvd, d, False) + _f8_matrix_bytes(F, d, True)
    # the converted weights are the only growth here (the (hi, lo) buffers already hold the operands)
    assert f8 - base == m.n_layers * per_layer
    # MoE: only q|k|v is converted
    x = configs.MIXTRAL
    gx = (D.workspace_bytes(x.replace(prefill_fp8=True), max_batch=16, max_prefill=512)
          - D.workspace_bytes(x, max_batch=16, max_prefill=512))
    assert gx == x.n_layers * _f8_matrix_bytes(x.q_dim + 2 * x.kv_dim, x.hidden, False)
    # prefills of at most 64 rows never take the form
    assert D.workspace_bytes(m.replace(prefill_fp8=True), 32, 64) == D.workspace_bytes(m, 32, 64)
    # an unknown form, and the form with fp32 weights, are refused
    c = D.make_config(m, 32, 4096)
    c.prefill_operands = 2
    assert _lib().dec_workspace_bytes(ctypes.byref(c)) == 0
    assert D.workspace_bytes(configs.TINY.replace(prefill_fp8=True, max_seq=256), 2, 128) == 0   # fp32 weights
    assert _create(configs.TINY, prefill_operands=1)[0] == D.DEC_ERR_INVALID
