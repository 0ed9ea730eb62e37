"""Matmul on the GPU: parity with the fp64 oracle, exact pins, bitwise row
invariance across M and row positions, bf16 == RNE(fp32)."""
import numpy as np
import pytest
import torch

import synth
from helpers import TOL_BF16, TOL_F32, bits_of, f64, poison_like, rel_err, to_dev

pytestmark = pytest.mark.gpu

M_SET = (1, 2, 7, 16, 64, 256, 512, 2048)


def _mm(a_bits, w_bits, f32=False, w_dev=None):
    import invariant_bi_matmul_amd as bi
    a = to_dev(a_bits)
    w = w_dev if w_dev is not None else to_dev(w_bits)
    dt = torch.float32 if f32 else torch.bfloat16
    c = poison_like(torch.empty(a.shape[0], w.shape[1], dtype=dt, device=a.device))
    bi.matmul(a, w, out=c, out_dtype=dt)
    return c.cpu().numpy() if f32 else bits_of(c)


@pytest.mark.parametrize("m", [1, 3, 8])
def test_toy_parity(orc, m):
    a, w = synth.matmul_inputs(m, 512, 256, seed=0)
    c = _mm(a, w)
    assert rel_err(f64(c), orc.matmul(a, w)) < TOL_BF16


@pytest.mark.parametrize("n", [4096, 14336])
def test_parity_full_size_sampled(orc, n):
    a, w = synth.matmul_inputs(2048, n, 4096, seed=0)
    wd = to_dev(w)
    c = _mm(a, None, w_dev=wd)
    cf = _mm(a, None, f32=True, w_dev=wd)
    pick = np.unique(np.concatenate([[0, 255, 256, 2047], synth.stream(1, "mmpick").integers(0, 2048, 20)]))
    ref = orc.matmul(a, w, rows=pick)
    assert rel_err(f64(c[pick]), ref) < TOL_BF16
    assert rel_err(cf[pick], ref) < TOL_F32
    # bf16 output is exactly the RNE of the fp32 output (same kernel, other store)
    assert np.array_equal(c, synth.bf16_bits(cf))


@pytest.mark.parametrize("n", [4096, 14336])
def test_row_invariance_across_m(n):
    a, w = synth.matmul_inputs(2048, n, 4096, seed=2)
    wd = to_dev(w)
    full = _mm(a, None, w_dev=wd)
    # the workload's M, M on both sides of the single-row-tile variants (A
    # loads for rows 0..63, 0..127, all 256; for the 64 x 32 tile's 128-wide
    # k-tiles rows 0..7, 0..15, 0..31, all 64, and its second wave idle up to
    # 32), and M that select each tile (N = 4096: 64 x 32 up to 128, 64 x 64 to
    # 256, 128 x 64 to 512, 128 x 128 to 1024, then the main tile; N = 14336:
    # 64 x 64 to 64, 128 x 128 to 256, the main tile to 1536, then 256 x 256)
    for m in list(M_SET[:-1]) + [8, 9, 17, 32, 33, 65, 100, 128, 129, 200, 255, 257, 513, 768,
                                 1024, 1025, 1536, 1537]:
        c = _mm(a[:m], None, w_dev=wd)
        assert np.array_equal(c, full[:m]), m
    # a row at many different positions inside tiles and batches
    perm = synth.stream(2, "mmperm").permutation(2048)
    cp = _mm(a[perm], None, w_dev=wd)
    assert np.array_equal(cp, full[perm])
    probe = a[1234:1235]
    for m in (1, 3, 300):
        others, _ = synth.matmul_inputs(m, 8, 4096, seed=50 + m)
        pos = m // 2
        batch = np.concatenate([others[:pos], probe, others[pos:]])
        cb = _mm(batch, None, w_dev=wd)
        assert np.array_equal(cb[pos], full[1234]), m


def test_integer_inputs_exact():
    g = np.random.default_rng(3)
    ai = g.integers(-4, 5, size=(300, 4096))
    wi = g.integers(-4, 5, size=(4096, 520))
    a = synth.bf16_bits(ai.astype(np.float32))
    w = synth.bf16_bits(wi.astype(np.float32))
    exact = (ai @ wi).astype(np.float64)  # |sum| <= 16*4096 < 2^24: exact in fp32
    cf = _mm(a, w, f32=True)
    assert np.array_equal(cf.astype(np.float64), exact)
    c = _mm(a, w)
    assert np.array_equal(c, synth.bf16_bits(exact.astype(np.float32)))


def test_one_hot_rows_select_w():
    _, w = synth.matmul_inputs(1, 4096, 4096, seed=4)
    idx = [0, 1, 63, 64, 2047, 4095]
    a = np.zeros((len(idx), 4096), dtype=np.uint16)
    for i, j in enumerate(idx):
        a[i, j] = 0x3F80  # bf16 1.0
    c = _mm(a, w)
    assert np.array_equal(c, w[idx])
    c0 = _mm(np.zeros((3, 4096), dtype=np.uint16), w, f32=True)
    assert np.all(c0 == 0.0) and not np.signbit(c0).any()


@pytest.mark.parametrize("m,n,k", [(5, 8, 64), (33, 264, 128), (257, 520, 192), (1, 4104, 256),
                                   (100, 264, 320), (64, 136, 64),
                                   # ragged in both M and N under each larger tile
                                   (500, 2056, 192), (1000, 2056, 128), (1100, 4104, 128),
                                   (2100, 4104, 128),
                                   # fewer k-tiles than the 256 x 256 tile's ring holds
                                   (2100, 4104, 64),
                                   # the 64 x 32 tile with 128-wide k-tiles (k % 128 == 0:
                                   # one k-tile; fewer than its ring; A rows 0..31 only)
                                   # and with 64-wide ones (k % 128 == 64)
                                   (2, 4104, 128), (17, 4104, 384), (9, 4104, 320)])
def test_ragged_shapes(orc, m, n, k):
    import invariant_bi_matmul_amd as bi
    tile = {(500, 2056): (128, 64), (1000, 2056): (128, 128), (1100, 4104): (256, 128),
            (2100, 4104): (256, 256)}
    if (m, n) in tile:
        assert bi.matmul_tile(m, n)[:2] == tile[(m, n)]
    a, w = synth.matmul_inputs(m, n, k, seed=5)
    c = _mm(a, w)
    assert rel_err(f64(c), orc.matmul(a, w)) < TOL_BF16
    cf = _mm(a, w, f32=True)
    assert rel_err(cf, orc.matmul(a, w)) < TOL_F32


def test_empty_and_k0():
    import invariant_bi_matmul_amd as bi
    w = torch.zeros(64, 16, dtype=torch.bfloat16, device="cuda")
    assert bi.matmul(torch.zeros(0, 64, dtype=torch.bfloat16, device="cuda"), w).shape == (0, 16)
    c = poison_like(torch.empty(4, 16, dtype=torch.float32, device="cuda"))
    bi.matmul(torch.zeros(4, 0, dtype=torch.bfloat16, device="cuda"),
              torch.zeros(0, 16, dtype=torch.bfloat16, device="cuda"), out=c, out_dtype=torch.float32)
    assert torch.all(c == 0).item()


def test_repeat_bitwise():
    a, w = synth.matmul_inputs(512, 14336, 4096, seed=6)
    wd = to_dev(w)
    c0 = _mm(a, None, w_dev=wd)
    for _ in range(20):
        assert np.array_equal(_mm(a, None, w_dev=wd), c0)


def test_pack_w_layout():
    import invariant_bi_matmul_amd as bi
    _, w = synth.matmul_inputs(1, 4128, 320, seed=7)
    wp = bi.matmul_pack_w(to_dev(w))
    expect = w.reshape(320, 4128 // 32, 32).transpose(1, 0, 2)
    assert np.array_equal(bits_of(wp), expect)


@pytest.mark.parametrize("m,n,k", [
    # every tile: 64 x 32 (128- and 64-wide k-tiles, row skipping), 64 x 64, 128 x 64,
    # 128 x 128, 256 x 128, 256 x 256, with N past the last full tile where n % 32 == 0
    (1, 4096, 4096), (9, 4096, 14336), (33, 4128, 320), (100, 4096, 256), (200, 4096, 192),
    (300, 4096, 128), (600, 4096, 128), (1100, 4096, 128), (2100, 4128, 128),
    (2048, 14336, 4096), (257, 2080, 128)])
def test_packed_equals_row_major(m, n, k):
    import invariant_bi_matmul_amd as bi
    a, w = synth.matmul_inputs(m, n, k, seed=8)
    wd = to_dev(w)
    ad = to_dev(a)
    wp = bi.matmul_pack_w(wd)
    for dt in (torch.bfloat16, torch.float32):
        ref = bi.matmul(ad, wd, out_dtype=dt)
        c = poison_like(torch.empty(m, n, dtype=dt, device=ad.device))
        bi.matmul_packed(ad, wp, out=c, out_dtype=dt)
        assert torch.equal(c.view(torch.int32 if dt == torch.float32 else torch.int16),
                           ref.view(torch.int32 if dt == torch.float32 else torch.int16)), (m, n, k, dt)


def test_packed_splitk_comparator_equals_row_major():
    import invariant_bi_matmul_amd as bi
    a, w = synth.matmul_inputs(16, 4096, 4096, seed=9)
    ad, wd = to_dev(a), to_dev(w)
    wp = bi.matmul_pack_w(wd)
    for s in (1, 4, 16):
        r = bi.bix_matmul_splitk(ad, wd, split_k=s)
        p = bi.bix_matmul_splitk(ad, wp, split_k=s)
        assert torch.equal(r.view(torch.int16), p.view(torch.int16)), s
