"""The library's calls replayed from a captured HIP graph give the eager
result, replay after replay, with eager work and synchronisation in between
(the bench times short launches this way).  No call allocates, clears or
copies behind the caller's back, so a capture holds only the kernels."""
import numpy as np
import pytest
import torch

import synth
from helpers import EPS, bits_of, dev, to_dev
import invariant_bi_matmul_amd as bi

pytestmark = pytest.mark.gpu


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replays_match(fn, outs, scramble):
    """Eager result, then three replays, each after scrambling the outputs
    eagerly; every replay must restore the eager bits."""
    fn()
    torch.cuda.synchronize()
    want = [bits_of(o) for o in outs]
    g = _capture(fn)
    for _ in range(3):
        scramble()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert np.array_equal(bits_of(o), w)


def test_rmsnorm_and_matmul_replay():
    x, g = synth.rmsnorm_inputs(300, 4096, seed=0)
    _, w = synth.matmul_inputs(1, 1024, 4096, seed=0)
    xd, gd, wd = to_dev(x), to_dev(g), to_dev(w)
    y = torch.empty_like(xd)
    c = torch.empty(300, 1024, dtype=torch.bfloat16, device=dev())

    def fn():
        bi.rmsnorm(xd, gd, EPS, out=y)
        bi.matmul(y, wd, out=c)

    _replays_match(fn, [y, c], lambda: (y.fill_(7.0), c.fill_(-3.0)))


def test_prefill_and_decode_replay():
    lens = [700, 300, 1200]
    prob = synth.attn_problem(lens, n_q=32, n_kv=8, d=128, seed=1)
    pool = synth.page_pool(lens, 8, 128, seed=2)
    kc, vc = to_dev(pool.k_pages), to_dev(pool.v_pages)
    bt = torch.from_numpy(pool.block_table).to(dev())
    # every sequence but its last token in one prefill, eagerly
    pre = [L - 1 for L in lens]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(pre)]), dtype=torch.int32, device=dev())
    cat = lambda a: to_dev(np.concatenate([a[b][:pre[b]] for b in range(3)]))
    bi.attn_prefill(cat(prob.q), cat(prob.k), cat(prob.v), cu,
                    torch.tensor(pre, dtype=torch.int32, device=dev()), bt, kc, vc, prob.scale,
                    max(pre))
    last = lambda a: to_dev(np.stack([a[b][lens[b] - 1] for b in range(3)]))
    q, kn, vn = last(prob.q), last(prob.k), last(prob.v)
    kvl = torch.tensor(lens, dtype=torch.int32, device=dev())
    o = torch.empty(3, 32, 128, dtype=torch.bfloat16, device=dev())
    lse = torch.empty(3, 32, dtype=torch.float32, device=dev())

    def fn():
        bi.attn_decode(q, kn, vn, kvl, bt, kc, vc, prob.scale, max(lens), out=o, lse=lse)

    _replays_match(fn, [o, lse], lambda: (o.fill_(1.0), lse.fill_(float("nan"))))
