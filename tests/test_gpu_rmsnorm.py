"""RMSNorm on the GPU: parity with the fp64 oracle, bitwise row invariance
across row counts and positions, pins, repeatability."""
import numpy as np
import pytest
import torch

import synth
from helpers import EPS, TOL_BF16, TOL_F32, bits_of, f64, poison_like, rel_err, to_dev

pytestmark = pytest.mark.gpu


def _run(x_bits, g_bits, eps=EPS):
    import invariant_bi_matmul_amd as bi
    x = to_dev(x_bits)
    y = poison_like(torch.empty_like(x))
    r = poison_like(torch.empty(x.shape[0], dtype=torch.float32, device=x.device))
    bi.rmsnorm(x, to_dev(g_bits), eps, out=y, rstd=r)
    return bits_of(y), r.cpu().numpy()


@pytest.mark.parametrize("rows", [1, 3, 8])
def test_toy_parity(orc, rows):
    x, g = synth.rmsnorm_inputs(rows, 256, seed=0)
    y, r = _run(x, g)
    yo, ro = orc.rmsnorm(x, g, EPS)
    assert rel_err(f64(y), yo) < TOL_BF16
    assert np.max(np.abs(r - ro) / ro) < TOL_F32


@pytest.mark.parametrize("hidden", [4096, 8192])
def test_parity_full_size_sampled(orc, hidden):
    x, g = synth.rmsnorm_inputs(16384, hidden, seed=0)
    y, r = _run(x, g)
    pick = np.unique(np.concatenate([[0, 1, 16383], synth.stream(0, "pick").integers(0, 16384, 61)]))
    yo, ro = orc.rmsnorm(x[pick], g, EPS)
    assert rel_err(f64(y[pick]), yo) < TOL_BF16
    assert np.max(np.abs(r[pick] - ro) / ro) < TOL_F32
    assert not np.isnan(r).any()


@pytest.mark.parametrize("hidden", [256, 4096, 8192])
def test_row_invariance_across_row_counts(hidden):
    full = 16384
    x, g = synth.rmsnorm_inputs(full, hidden, seed=1)
    y_full, r_full = _run(x, g)
    for rows in (1, 2, 3, 7, 16, 255, 256, 1000, 4096, 16383):
        y, r = _run(x[:rows], g)
        assert np.array_equal(y, y_full[:rows]), rows
        assert np.array_equal(r.view(np.uint32), r_full[:rows].view(np.uint32)), rows


def test_probe_position_and_companions():
    x, g = synth.rmsnorm_inputs(512, 4096, seed=2)
    y, _ = _run(x, g)
    perm = synth.stream(2, "perm").permutation(512)
    yp, _ = _run(x[perm], g)
    assert np.array_equal(yp, y[perm])
    # probe row alone vs between unrelated companions
    other, _ = synth.rmsnorm_inputs(64, 4096, seed=3)
    batch = np.concatenate([other[:37], x[5:6], other[37:]])
    yb, _ = _run(batch, g)
    assert np.array_equal(yb[37], y[5])


def test_in_place_equals_out_of_place():
    import invariant_bi_matmul_amd as bi
    x, g = synth.rmsnorm_inputs(300, 4096, seed=4)
    y, _ = _run(x, g)
    xt = to_dev(x)
    bi.rmsnorm(xt, to_dev(g), EPS, out=xt)
    assert np.array_equal(bits_of(xt), y)


def test_epilogue_matches_rstd_bitwise():
    """y == bf16((x * rstd) * gamma) with two fp32 roundings, from the exported rstd."""
    x, g = synth.rmsnorm_inputs(257, 4096, seed=5)
    y, r = _run(x, g)
    t = (synth.bf16_to_f32(x) * r[:, None].astype(np.float32)).astype(np.float32)
    t = (t * synth.bf16_to_f32(g)[None, :]).astype(np.float32)
    assert np.array_equal(y, synth.bf16_bits(t))


def test_pins():
    H = 4096
    one = synth.bf16_bits(np.float32(1.0))
    ones_g = np.full(H, one, dtype=np.uint16)
    # rows of +-1 with gamma = 1: y == x bitwise (1/sqrt(1+1e-6) rounds to 1 in bf16)
    signs = synth.stream(6, "signs").integers(0, 2, size=(4, H)).astype(np.float32) * 2 - 1
    xs = synth.bf16_bits(signs)
    y, _ = _run(xs, ones_g)
    assert np.array_equal(y, xs)
    # zero row: y = 0, rstd = 1/sqrt(eps)
    y, r = _run(np.zeros((2, H), dtype=np.uint16), ones_g)
    assert np.all(f64(y) == 0.0)
    np.testing.assert_allclose(r, 1.0 / np.sqrt(EPS), rtol=1e-6)
    # constant row c: y = c / sqrt(c^2 + eps) * gamma
    _, g = synth.rmsnorm_inputs(1, H, seed=7)
    for c in (1e-3, 0.5, -3.0, 40.0):
        cb = synth.bf16_bits(np.float32(c))
        y, r = _run(np.full((1, H), cb, dtype=np.uint16), g)
        cv = f64(cb)
        expect = cv / np.sqrt(cv * cv + EPS) * f64(g)
        assert rel_err(f64(y[0]), expect) < TOL_BF16
        np.testing.assert_allclose(r[0], 1.0 / np.sqrt(cv * cv + EPS), rtol=TOL_F32)


def test_repeat_bitwise():
    x, g = synth.rmsnorm_inputs(1024, 8192, seed=8)
    y0, r0 = _run(x, g)
    for _ in range(20):
        y, r = _run(x, g)
        assert np.array_equal(y, y0) and np.array_equal(r.view(np.uint32), r0.view(np.uint32))


def test_zero_rows_is_noop():
    import invariant_bi_matmul_amd as bi
    x = torch.empty(0, 4096, dtype=torch.bfloat16, device="cuda")
    g = to_dev(np.zeros(4096, dtype=np.uint16))
    assert bi.rmsnorm(x, g).shape == (0, 4096)
