"""Pins for the error-compensated matmul oracle (``oracle.ec``): the split's
closed forms and error bound, and the product's dropped lo*lo term.  CPU only."""
import numpy as np

from oracle import ec


def test_split_closed_forms():
    x = np.array([1.0, 1 + 2 ** -9, 1 + 2 ** -10 + 2 ** -14, -3.0 - 2 ** -12, 0.0],
                 dtype=np.float32)
    hi, lo = ec.split(x)
    # 1 + 2^-9 is below half an ulp of bf16 at 1 (2^-8): hi = 1, lo = 2^-9
    assert hi.tolist() == [1.0, 1.0, 1.0, -3.0, 0.0]
    assert lo.tolist() == [0.0, 2 ** -9, 2 ** -10 + 2 ** -14, -2 ** -12, 0.0]
    # above half an ulp rounds hi up and makes lo negative
    hi, lo = ec.split(np.array([1 + 2 ** -8 + 2 ** -12], dtype=np.float32))
    assert hi[0] == 1 + 2 ** -7 and lo[0] == -(2 ** -8) + 2 ** -12


def test_split_error_bound_and_specials():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10.0 ** rng.integers(-20, 20, 100000)).astype(np.float32)
    hi, lo = ec.split(x)
    xd = x.astype(np.float64)
    # two bf16 halves carry 16 significant bits: |x - hi - lo| <= 2^-16 |x|
    assert np.all(np.abs(xd - hi - lo) <= 2.0 ** -16 * np.abs(xd))
    hi, lo = ec.split(np.array([np.inf, -np.inf, np.nan], dtype=np.float32))
    assert hi[0] == np.inf and hi[1] == -np.inf and np.isnan(hi[2])
    assert lo.tolist() == [0.0, 0.0, 0.0]


def test_product_drops_only_lo_lo():
    a = np.array([[1 + 2 ** -9, 2.0]], dtype=np.float32)
    w = np.array([[1 + 2 ** -9], [3.0]], dtype=np.float32)
    # exact: (1 + 2^-9)^2 + 6 = 7 + 2^-8 + 2^-18; compensated drops 2^-9 * 2^-9
    assert ec.exact(a, w)[0, 0] == 7 + 2 ** -8 + 2 ** -18
    assert ec.ec_product(a, w)[0, 0] == 7 + 2 ** -8
    # bf16-representable operands: lo = 0 and the product is exact
    b = np.array([[1.5, -2.0, 0.25]], dtype=np.float32)
    v = np.array([[4.0], [0.5], [-8.0]], dtype=np.float32)
    assert ec.ec_product(b, v)[0, 0] == ec.exact(b, v)[0, 0] == 3.0


def test_compensation_beats_bf16_on_random_operands():
    rng = np.random.default_rng(1)
    a = rng.standard_normal((8, 512)).astype(np.float32)
    w = rng.standard_normal((512, 64)).astype(np.float32)
    ref = ec.exact(a, w)
    ah, _ = ec.split(a)
    wh, _ = ec.split(w)
    err_bf16 = np.abs(ah @ wh - ref).max() / np.abs(ref).max()
    err_ec = np.abs(ec.ec_product(a, w) - ref).max() / np.abs(ref).max()
    assert err_ec < 1e-5 < 1e-3 < err_bf16 * 10
    assert err_ec * 100 < err_bf16
