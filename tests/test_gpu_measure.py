"""The measurement kernels behind the bench's ceilings: they run, write
nothing, and reject sizes they cannot read in 16-byte loads."""
import pytest
import torch

import invariant_bi_matmul_amd as bi

pytestmark = pytest.mark.gpu


def test_read_stream_reads_and_writes_nothing():
    x = torch.arange(1 << 18, dtype=torch.int32, device="cuda")   # 1 MiB
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for wg in (1, 7, 256, 2048):
        assert bi.bix_read_stream(x, wg, sink) == 1 << 20
    # a tail shorter than one grid stride and a tensor smaller than one stride
    assert bi.bix_read_stream(x[:1000 * 4], 2048, sink) == 16000
    torch.cuda.synchronize()
    assert sink.tolist() == [0, 0, 0, 0]


def test_read_stream_rejects_ragged_sizes():
    x = torch.zeros(5, dtype=torch.int32, device="cuda")   # 20 bytes
    with pytest.raises(bi.BIError):
        bi.bix_read_stream(x, 1)
    with pytest.raises(bi.BIError):
        bi.bix_read_stream(torch.zeros(8, dtype=torch.int32, device="cuda")[1:5], 1)


def test_mfma_loop_runs_and_writes_nothing():
    sink = torch.zeros(4, dtype=torch.float32, device="cuda")
    assert bi.bix_mfma_loop(100, 512, sink) == 4.0 * 4 * 32768 * 100 * 512
    assert bi.bix_mfma_loop(0, 512, sink) == 0.0
    torch.cuda.synchronize()
    assert sink.tolist() == [0.0, 0.0, 0.0, 0.0]
