"""Negative controls: the non-invariant comparators (split-row RMSNorm,
split-K matmul, batch-dependent split-KV decode) stay within tolerance of the
oracle but change bits with the batch -- which shows the invariance tests can
see a non-invariant kernel."""
import numpy as np
import pytest
import torch

import synth
from helpers import EPS, TOL_BF16, PagedRun, bits_of, f64, oracle_attention, rel_err, to_dev

pytestmark = pytest.mark.gpu


def test_splitrow_rmsnorm_depends_on_row_count(orc):
    """Split-row RMSNorm: a row's fp32 sum of squares (seen through rstd) or
    its bf16 output changes with the number of rows in the call."""
    import invariant_bi_matmul_amd as bi
    rows = 4096
    x, g = synth.rmsnorm_inputs(rows, 8192, seed=0)
    gd = to_dev(g)
    r_full = torch.empty(rows, dtype=torch.float32, device="cuda")
    full = bits_of(bi.bix_rmsnorm_splitrow(to_dev(x), gd, EPS, rstd=r_full)[0])
    r_full = r_full.cpu().numpy()
    differs = 0
    for i in range(128):
        r1 = torch.empty(1, dtype=torch.float32, device="cuda")
        one = bits_of(bi.bix_rmsnorm_splitrow(to_dev(x[i:i + 1]), gd, EPS, rstd=r1)[0])
        same = np.array_equal(one[0], full[i]) and \
            r1.cpu().numpy().view(np.uint32)[0] == r_full.view(np.uint32)[i]
        differs += int(not same)
        if i < 8:
            yo, _ = orc.rmsnorm(x[i:i + 1], g, EPS)
            assert rel_err(f64(one), yo) < TOL_BF16
    assert differs > 0
    # the invariant kernel gives bitwise the same row and rstd alone
    ya, ra = bi.rmsnorm(to_dev(x), gd, EPS, with_rstd=True)
    yb, rb = bi.rmsnorm(to_dev(x[:1]), gd, EPS, with_rstd=True)
    assert np.array_equal(bits_of(yb)[0], bits_of(ya)[0])
    assert ra[0].item() == rb[0].item()


def test_splitk_matmul_depends_on_m(orc):
    import invariant_bi_matmul_amd as bi
    a, w = synth.matmul_inputs(2048, 4096, 4096, seed=1)
    wd = to_dev(w)
    full = bits_of(bi.bix_matmul_splitk(to_dev(a), wd))
    small = bits_of(bi.bix_matmul_splitk(to_dev(a[:8]), wd))
    assert not np.array_equal(small, full[:8])
    assert rel_err(f64(small), orc.matmul(a, w, rows=range(8))) < TOL_BF16


def test_splitkv_decode_depends_on_batch(orc):
    L = 4096
    comp, _ = synth.ragged_lengths(63, 4096, seed=2)
    outs = []
    for lens, tags, pb in (([L], ["probe"], 0),
                           ([L] + comp, ["probe"] + ["c%d" % i for i in range(63)], 0)):
        prob = synth.attn_problem(lens, n_q=32, n_kv=8, d=128, seed=3, tags=tags)
        run = PagedRun(prob, page_seed=1)
        run.prefill([(b, n - 1) for b, n in enumerate(lens)])
        run.decode(list(range(len(lens))), comparator=True)
        outs.append(run.out[pb][L - 1].copy())
        o, _ = oracle_attention(orc, prob, [(pb, L - 1)])
        assert rel_err(f64(run.out[pb][L - 1]), o[0]) < TOL_BF16
    assert not np.array_equal(outs[0], outs[1])
