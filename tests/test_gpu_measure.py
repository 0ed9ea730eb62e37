"""The measurement kernels behind the bench's ceilings: they run, write
nothing, and reject sizes they cannot read in 16-byte loads."""
import pytest
import torch

import invariant_bi_matmul_amd as bi

pytestmark = pytest.mark.gpu


def test_read_stream_reads_and_writes_nothing():
    x = torch.arange(1 << 18, dtype=torch.int32, device="cuda")   # 1 MiB = 128 chunks
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for wg in (1, 7, 64, 256, 2048):
        assert bi.bix_read_stream(x, wg, sink) == 1 << 20
    # fewer chunks than a wave's ring, and fewer than waves
    assert bi.bix_read_stream(x[:3 * 2048], 1, sink) == 3 * 8192
    assert bi.bix_read_stream(x[:3 * 2048], 256, sink) == 3 * 8192
    torch.cuda.synchronize()
    assert sink.tolist() == [0, 0, 0, 0]


def test_read_stream_rejects_ragged_sizes():
    with pytest.raises(bi.BIError):   # 16000 bytes: not whole 8 KiB chunks
        bi.bix_read_stream(torch.zeros(4000, dtype=torch.int32, device="cuda"), 1)
    with pytest.raises(bi.BIError):   # misaligned
        bi.bix_read_stream(torch.zeros(2049 * 4, dtype=torch.int32, device="cuda")[1:2049], 1)


def test_mfma_loop_runs_and_writes_nothing():
    sink = torch.zeros(4, dtype=torch.float32, device="cuda")
    assert bi.bix_mfma_loop(100, 512, sink) == 4.0 * 4 * 32768 * 100 * 512
    assert bi.bix_mfma_loop(0, 512, sink) == 0.0
    assert bi.bix_mfma_loop(101, 512, sink, varied=True) == 4.0 * 4 * 32768 * 101 * 512
    torch.cuda.synchronize()
    assert sink.tolist() == [0.0, 0.0, 0.0, 0.0]
