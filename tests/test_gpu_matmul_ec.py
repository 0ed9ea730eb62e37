"""Error-compensated matmul on the GPU: the packed weight against the
oracle's split (bitwise), the product against the oracle's formula and the
exact product element by element, the bf16-operand path, and the rows'
invariance across M.

Bounds.  hi = bf16(x) is within 2^-8 |x| of x, and lo = bf16(x - hi) within
2^-8 |x - hi| <= 2^-16 |x| of x - hi; so x = hi + lo + r with |lo| <= 2^-8 |x|
(to first order) and |r| <= 2^-16 |x|.  The three products then miss a w by
hi r' + lo (lo' + r') + r w, at most about 3 * 2^-16 |a||w| per term.  Each
element is held to 2^-14 sum_k |a_ik||w_kj|: that bound plus room for the
fp32 accumulation, whose error grows with the partial sums (about sqrt(k)
times a term) rather than with sum |a||w| and stays far below it here.  A
plain bf16 product misses each term by up to 2^-7 |a||w| and breaks the
bound.  The element-wise relative error (|g - o| / max(|o|, rms(row)), the
metric used throughout) is held to 1e-4, the bar for fp32-accumulated
results, where a plain bf16 product is near 2^-8."""
import numpy as np
import pytest
import torch

import synth
from helpers import TOL_F32, dev, rel_err
import invariant_bi_matmul_amd as bi
from oracle import ec

pytestmark = pytest.mark.gpu


def _f32(shape, seed, tag, scale=1.0):
    return (synth.stream(seed, tag).standard_normal(shape) * scale).astype(np.float32)


def _abs_bound(a, w):
    """2^-14 sum_k |a_ik| |w_kj| for every element."""
    return np.abs(a.astype(np.float64)) @ np.abs(w.astype(np.float64)) * 2.0 ** -14


def test_pack_w_is_hi_lo_hi_exactly():
    w = _f32((128, 64), 0, "ec.w", 3.0)
    w[0, :4] = [np.inf, -np.inf, np.nan, 0.0]
    w3 = bi.matmul_ec_pack_w(torch.from_numpy(w).to(dev()))
    got = w3.float().cpu().numpy().astype(np.float64)
    hi, lo = ec.split(w)
    assert np.array_equal(got[:128], hi, equal_nan=True)
    assert np.array_equal(got[128:256], lo, equal_nan=True)
    assert np.array_equal(got[256:], hi, equal_nan=True)


@pytest.mark.parametrize("m,k,n", [(1, 256, 512), (7, 256, 512), (300, 4096, 520),
                                   (513, 1024, 776)])
def test_ec_parity(m, k, n):
    a = _f32((m, k), 1, "ec.a")
    w = _f32((k, n), 1, "ec.w", 1.0 / np.sqrt(k))
    w3 = bi.matmul_ec_pack_w(torch.from_numpy(w).to(dev()))
    c = bi.matmul_ec(torch.from_numpy(a).to(dev()), w3).cpu().numpy().astype(np.float64)
    # the formula, up to fp32 accumulation
    assert rel_err(c, ec.ec_product(a, w)) < TOL_F32
    # the exact product: element-wise, and within the split's analytic bound
    exact = ec.exact(a, w)
    err_ec = rel_err(c, exact)
    assert err_ec < TOL_F32
    bound = _abs_bound(a, w)
    assert np.all(np.abs(c - exact) <= bound)
    # a plain bf16 product of the same operands is far less accurate
    plain = bi.matmul(torch.from_numpy(a).to(dev()).to(torch.bfloat16),
                      torch.from_numpy(w).to(dev()).to(torch.bfloat16),
                      out_dtype=torch.float32).cpu().numpy().astype(np.float64)
    assert err_ec * 20 < rel_err(plain, exact)
    if k >= 1024:
        assert not np.all(np.abs(plain - exact) <= bound)


def test_ec_at_the_large_matmul_shape_on_sampled_rows():
    """2048 x 4096 x 14336 (the largest matmul of the workload), fp32
    operands; 24 rows checked against the exact product element by element."""
    m, k, n = 2048, 4096, 14336
    g = torch.Generator(device=dev())
    g.manual_seed(11)
    a = torch.randn(m, k, device=dev(), generator=g)
    w = torch.randn(k, n, device=dev(), generator=g) / 64.0
    w3 = bi.matmul_ec_pack_w(w)
    c = bi.matmul_ec(a, w3)
    rows = np.sort(synth.stream(0, "ec.rows").choice(m, size=24, replace=False))
    a_h, w_h = a[rows].cpu().numpy(), w.cpu().numpy()
    exact = ec.exact(a_h, w_h)
    got = c[rows].cpu().numpy().astype(np.float64)
    assert rel_err(got, exact) < TOL_F32
    assert np.all(np.abs(got - exact) <= _abs_bound(a_h, w_h))


def test_bf16_operand_takes_two_products_with_the_same_sum():
    """A bf16 operand has lo = 0: its call runs [a | a] against [hi; lo] and
    gives the fp32-operand call's bits on the same values; its bf16 output is
    the round-to-nearest-even of the fp32 one."""
    m, k, n = 77, 2048, 1032
    a16 = torch.from_numpy(_f32((m, k), 3, "ec.a16")).to(dev()).to(torch.bfloat16)
    w = _f32((k, n), 3, "ec.w16", 1.0 / np.sqrt(k))
    w3 = bi.matmul_ec_pack_w(torch.from_numpy(w).to(dev()))
    c2 = bi.matmul_ec(a16, w3)
    c3 = bi.matmul_ec(a16.float(), w3)
    assert torch.equal(c2.view(torch.int32), c3.view(torch.int32))
    cb = bi.matmul_ec(a16, w3, out_dtype=torch.bfloat16)
    assert torch.equal(cb.view(torch.int16), c2.to(torch.bfloat16).view(torch.int16))
    a_h = a16.float().cpu().numpy()
    exact = ec.exact(a_h, w)
    got = c2.cpu().numpy().astype(np.float64)
    assert rel_err(got, exact) < TOL_F32
    assert np.all(np.abs(got - exact) <= _abs_bound(a_h, w))


def test_ec_rows_are_invariant_across_m():
    k, n = 1024, 640
    a = _f32((513, k), 2, "ec.a2")
    w3 = bi.matmul_ec_pack_w(torch.from_numpy(_f32((k, n), 2, "ec.w2", 1 / 32)).to(dev()))
    for dt in (torch.float32, torch.bfloat16):
        full = bi.matmul_ec(torch.from_numpy(a).to(dev()).to(dt), w3)
        for m in (1, 2, 17, 256, 257):
            part = bi.matmul_ec(torch.from_numpy(a[:m]).to(dev()).to(dt), w3)
            assert torch.equal(part.view(torch.int32), full[:m].view(torch.int32)), (dt, m)
        probe = bi.matmul_ec(torch.from_numpy(a[400:401]).to(dev()).to(dt), w3)
        assert torch.equal(probe.view(torch.int32), full[400:401].view(torch.int32))
