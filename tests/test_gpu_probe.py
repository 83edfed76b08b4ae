"""The measured-ceiling probes (libdec_probe.so, include/dec_probe.h) that
bench.py reports beside the published peaks: the streaming read touches every
word once (its per-thread XOR equals the host's), the copy is exact, and the
rates are plausible for one MI355X."""
import numpy as np
import pytest
import torch

from decoder_only_forward_amd import probe

pytestmark = pytest.mark.gpu


def test_stream_read_reads_every_word_once():
    g = torch.Generator().manual_seed(7)
    host = torch.randint(-2**31, 2**31 - 1, (16 << 20,), dtype=torch.int32, generator=g)   # 64 MiB
    buf = host.cuda()
    runs = buf.numel() * 4 // probe.RUN_BYTES
    sink = torch.zeros(runs, dtype=torch.int32, device="cuda")
    ms = probe.stream_read(buf, reps=2, sink=sink)
    assert ms > 0
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32).reshape(runs, -1), axis=1)
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), want)


def test_copy_is_exact():
    src = torch.randint(0, 255, (32 << 20,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros_like(src)
    assert probe.copy(src, dst, reps=2) > 0
    assert torch.equal(src, dst)


def test_rates_are_plausible():
    buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    read = buf.numel() / (probe.stream_read(buf, reps=3) * 1e-3) / 1e9
    ms, fl = probe.mfma_bf16(iters=1024, reps=3)
    tflops = fl / (ms * 1e-3) / 1e12
    print(f"read {read:.0f} GB/s, bf16 MFMA {tflops:.0f} TFLOP/s")
    assert 1000 < read < 12000
    assert 100 < tflops < 2600
