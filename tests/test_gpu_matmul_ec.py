"""Error-compensated matmul on the GPU: the packed weight against the
oracle's split (bitwise), the product against the oracle's formula and the
exact product, and the rows' invariance across M."""
import numpy as np
import pytest
import torch

import synth
from helpers import TOL_F32, dev
import invariant_bi_matmul_amd as bi
from oracle import ec

pytestmark = pytest.mark.gpu


def _f32(shape, seed, tag, scale=1.0):
    return (synth.stream(seed, tag).standard_normal(shape) * scale).astype(np.float32)


def _rel(got, ref):
    return float(np.abs(np.asarray(got, np.float64) - ref).max() / np.abs(ref).max())


def test_pack_w_is_hi_lo_hi_exactly():
    w = _f32((128, 64), 0, "ec.w", 3.0)
    w[0, :4] = [np.inf, -np.inf, np.nan, 0.0]
    w3 = bi.matmul_ec_pack_w(torch.from_numpy(w).to(dev()))
    got = w3.float().cpu().numpy().astype(np.float64)
    hi, lo = ec.split(w)
    assert np.array_equal(got[:128], hi, equal_nan=True)
    assert np.array_equal(got[128:256], lo, equal_nan=True)
    assert np.array_equal(got[256:], hi, equal_nan=True)


@pytest.mark.parametrize("m,k,n", [(1, 256, 512), (7, 256, 512), (300, 4096, 520)])
def test_ec_parity(m, k, n):
    a = _f32((m, k), 1, "ec.a")
    w = _f32((k, n), 1, "ec.w", 1.0 / np.sqrt(k))
    w3 = bi.matmul_ec_pack_w(torch.from_numpy(w).to(dev()))
    c = bi.matmul_ec(torch.from_numpy(a).to(dev()), w3).cpu().numpy()
    # the formula up to fp32 accumulation, and the exact product up to lo*lo
    assert _rel(c, ec.ec_product(a, w)) < TOL_F32
    exact = ec.exact(a, w)
    err_ec = _rel(c, exact)
    assert err_ec < TOL_F32
    # a plain bf16 product of the same operands is far less accurate
    plain = bi.matmul(torch.from_numpy(a).to(dev()).to(torch.bfloat16),
                      torch.from_numpy(w).to(dev()).to(torch.bfloat16),
                      out_dtype=torch.float32).cpu().numpy()
    assert err_ec * 20 < _rel(plain, exact)


def test_ec_rows_are_invariant_across_m():
    k, n = 1024, 640
    a = _f32((513, k), 2, "ec.a2")
    w3 = bi.matmul_ec_pack_w(torch.from_numpy(_f32((k, n), 2, "ec.w2", 1 / 32)).to(dev()))
    full = bi.matmul_ec(torch.from_numpy(a).to(dev()), w3)
    for m in (1, 2, 17, 256, 257):
        part = bi.matmul_ec(torch.from_numpy(a[:m]).to(dev()), w3)
        assert torch.equal(part.view(torch.int32), full[:m].view(torch.int32)), m
    probe = bi.matmul_ec(torch.from_numpy(a[400:401]).to(dev()), w3)
    assert torch.equal(probe.view(torch.int32), full[400:401].view(torch.int32))
