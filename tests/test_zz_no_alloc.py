"""bi_attn_decode_noalloc: decode whose split partials live in the library's
own per-GPU scratch array instead of a caller's workspace.  Called through the
C ABI (ctypes binding) and checked bit for bit against bi_attn_decode on the
same inputs -- outputs, lse and the appended cache -- on two calls in a row,
the second smaller than the first, so stale records of the first call sit in
the array during the second.  Also: a size beyond the array is refused with
nothing enqueued."""
import numpy as np
import pytest
import torch

import invariant_bi_matmul_amd as bi
import synth
from helpers import bits_of, dev, f64, lse_err, oracle_attention, rel_err, to_dev, TOL_BF16, TOL_F32

pytestmark = pytest.mark.gpu


def _case(lens, nq, nkv, d, tag):
    """Sequences whose caches hold positions 0..L-2; the call brings L-1."""
    prob = synth.attn_problem(lens, nq, nkv, d, seed=3,
                              tags=["%s%d" % (tag, b) for b in range(len(lens))])
    pool = synth.page_pool(lens, nkv, d, seed=5)
    for b, L in enumerate(lens):
        synth.scatter_tokens(pool, b, 0, prob.k[b][:L - 1], prob.v[b][:L - 1])
    pick = lambda xs: np.stack([x[L - 1] for x, L in zip(xs, lens)])
    return prob, pool, pick(prob.q), pick(prob.k), pick(prob.v)


def _run(noalloc, prob, pool, q, kn, vn):
    kc, vc = to_dev(pool.k_pages), to_dev(pool.v_pages)
    bt = torch.from_numpy(pool.block_table).to(dev())
    kvl = torch.tensor(prob.lens, dtype=torch.int32, device=dev())
    out = torch.full((len(prob.lens), prob.n_q, prob.d), float("nan"), dtype=torch.bfloat16,
                     device=dev())
    lse = torch.full((len(prob.lens), prob.n_q), float("nan"), dtype=torch.float32, device=dev())
    args = (to_dev(q), to_dev(kn), to_dev(vn), kvl, bt, kc, vc, prob.scale, max(prob.lens))
    if noalloc:
        bi.attn_decode_noalloc(*args, out=out, lse=lse)
    else:
        need = bi.attn_workspace_bytes(
            bi.make_shape(len(prob.lens), prob.n_q, prob.n_kv, prob.d, bt.shape[1], kc.shape[0],
                          prob.scale), len(prob.lens), max(prob.lens))
        ws = torch.full((need // 4 + 4,), float("nan"), dtype=torch.float32, device=dev())
        bi.attn_decode(*args, workspace=ws, out=out, lse=lse)
    torch.cuda.synchronize()
    return bits_of(out), lse.cpu().numpy(), bits_of(kc), bits_of(vc)


def test_noalloc_equals_decode_on_two_calls_in_a_row(orc):
    cases = [
        # first: 40 ragged sequences up to 3000 positions, GQA 32/8, d=128
        (synth.ragged_lengths(40, 3000, seed=11)[0], 32, 8, 128, "big"),
        # then a smaller call: 3 sequences, GQA 4/4, d=64
        ([300, 17, 257], 4, 4, 64, "small"),
    ]
    for lens, nq, nkv, d, tag in cases:
        print("noalloc case %s: B=%d max_len=%d nq=%d nkv=%d d=%d" %
              (tag, len(lens), max(lens), nq, nkv, d), flush=True)
        prob, pool, q, kn, vn = _case(lens, nq, nkv, d, tag)
        ref = _run(False, prob, pool, q, kn, vn)
        got = _run(True, prob, pool, q, kn, vn)
        for name, r, g in zip(("out", "lse", "k_cache", "v_cache"), ref, got):
            assert np.array_equal(r.view(np.uint8), g.view(np.uint8)), (tag, name)
        picks = [(b, L - 1) for b, L in enumerate(lens)]
        oo, ol = oracle_attention(orc, prob, picks)
        assert rel_err(f64(got[0]), oo) < TOL_BF16, tag
        assert lse_err(got[1], ol) < TOL_F32, tag


def test_noalloc_refuses_a_call_beyond_its_array():
    B, nq, nkv, d, L = 64, 32, 8, 128, 32768
    shape = bi.make_shape(B, nq, nkv, d, L // 16, 8, float(np.float32(d ** -0.5)))
    assert bi.attn_workspace_bytes(shape, B, L) > bi.DECODE_SCRATCH_BYTES
    kc = torch.zeros(8, nkv, 16, d, dtype=torch.bfloat16, device=dev())
    vc = torch.zeros_like(kc)
    bt = torch.zeros(B, L // 16, dtype=torch.int32, device=dev())
    kvl = torch.full((B,), L, dtype=torch.int32, device=dev())
    q = torch.zeros(B, nq, d, dtype=torch.bfloat16, device=dev())
    kn = torch.ones(B, nkv, d, dtype=torch.bfloat16, device=dev())
    out = torch.full_like(q, float("nan"))
    with pytest.raises(bi.BIError) as e:
        bi.attn_decode_noalloc(q, kn, kn, kvl, bt, kc, vc, 0.088388346, L, out=out)
    assert e.value.status == 4  # BI_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()          # nothing ran
    assert int(torch.count_nonzero(kc)) == 0       # nothing was appended
