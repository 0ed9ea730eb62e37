"""The debug build (libbi_debug.so): attention calls check their device index
arrays before launching.  A valid call gives the release library's bits; a
bad block-table entry, a length past the bound or a broken cu_q is reported
as BI_ERR_INVALID_SHAPE with nothing launched (the outputs keep their
poison).  The check kernel reads only inside the arrays the shape
describes, so no bad entry is ever followed."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from helpers import bits_of, dev, to_dev
import invariant_bi_matmul_amd as bi

pytestmark = pytest.mark.gpu
SHAPE_ERR = 2


@pytest.fixture(scope="module")
def dbg():
    return bi.load_library(bi.debug_lib_path())


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


class Case:
    """Three sequences (GQA 8/2, d=128): prefill all but the last token
    through the release library, then the decode inputs for the last one."""

    def __init__(self):
        self.lens = [300, 17, 520]
        prob = synth.attn_problem(self.lens, n_q=8, n_kv=2, d=128, seed=5)
        self.prob = prob
        pool = synth.page_pool(self.lens, 2, 128, seed=6)
        self.P = pool.k_pages.shape[0]
        self.kc, self.vc = to_dev(pool.k_pages), to_dev(pool.v_pages)
        self.bt_host = pool.block_table.copy()
        self.maxp = self.bt_host.shape[1]
        pre = [L - 1 for L in self.lens]
        cat = lambda a: to_dev(np.concatenate([a[b][:pre[b]] for b in range(3)]))
        self.cu = torch.tensor(np.concatenate([[0], np.cumsum(pre)]), dtype=torch.int32,
                               device=dev())
        self.pre_args = (cat(prob.q), cat(prob.k), cat(prob.v))
        self.pre = pre
        bi.attn_prefill(*self.pre_args, self.cu, torch.tensor(pre, dtype=torch.int32,
                                                              device=dev()),
                        torch.from_numpy(self.bt_host).to(dev()), self.kc, self.vc, prob.scale,
                        max(pre))
        last = lambda a: to_dev(np.stack([a[b][self.lens[b] - 1] for b in range(3)]))
        self.q, self.kn, self.vn = last(prob.q), last(prob.k), last(prob.v)
        self.shape = bi.make_shape(3, 8, 2, 128, self.maxp, self.P, prob.scale)
        self.ws_bytes = bi.attn_workspace_bytes(self.shape, 3, max(self.lens))
        self.ws = torch.empty(self.ws_bytes // 4 + 4, dtype=torch.float32, device=dev())

    def decode(self, lib, kv_len, bt, max_kv_len):
        out = torch.full((3, 8, 128), float("nan"), dtype=torch.bfloat16, device=dev())
        st = lib.bi_attn_decode(ctypes.byref(self.shape), _p(self.q), _p(self.kn), _p(self.vn),
                                _p(kv_len), _p(bt), _p(self.kc), _p(self.vc), _p(out), None,
                                max_kv_len, _p(self.ws), self.ws_bytes, _stream())
        torch.cuda.synchronize()
        return st, out


def test_valid_decode_matches_release(dbg):
    c = Case()
    kvl = torch.tensor(c.lens, dtype=torch.int32, device=dev())
    bt = torch.from_numpy(c.bt_host).to(dev())
    st, out_dbg = c.decode(dbg, kvl, bt, max(c.lens))
    assert st == 0
    st, out_rel = c.decode(bi.load(), kvl, bt, max(c.lens))
    assert st == 0
    assert np.array_equal(bits_of(out_dbg), bits_of(out_rel))


def test_bad_tables_are_reported_before_any_launch(dbg):
    c = Case()
    good = torch.tensor(c.lens, dtype=torch.int32, device=dev())
    # a block-table entry past the pool, in a page the sequence reaches
    bad_bt = c.bt_host.copy()
    bad_bt[2, 5] = c.P + 7
    st, out = c.decode(dbg, good, torch.from_numpy(bad_bt).to(dev()), max(c.lens))
    assert st == SHAPE_ERR and torch.isnan(out.float()).all()
    # a negative entry
    bad_bt = c.bt_host.copy()
    bad_bt[1, 0] = -1
    st, out = c.decode(dbg, good, torch.from_numpy(bad_bt).to(dev()), max(c.lens))
    assert st == SHAPE_ERR and torch.isnan(out.float()).all()
    # a length past max_kv_len, and a zero length
    bt = torch.from_numpy(c.bt_host).to(dev())
    for lens in ([300, 17, 521], [300, 0, 520]):
        st, out = c.decode(dbg, torch.tensor(lens, dtype=torch.int32, device=dev()), bt, 520)
        assert st == SHAPE_ERR and torch.isnan(out.float()).all(), lens
    # an entry past the sequence's last page is not looked at
    ok_bt = c.bt_host.copy()
    ok_bt[1, 3:] = c.P + 100
    st, _ = c.decode(dbg, good, torch.from_numpy(ok_bt).to(dev()), max(c.lens))
    assert st == 0


def test_bad_query_ranges_are_reported(dbg):
    c = Case()
    q, k, v = c.pre_args
    kvl = torch.tensor(c.pre, dtype=torch.int32, device=dev())
    bt = torch.from_numpy(c.bt_host).to(dev())
    T = q.shape[0]
    for cu in ([0, 299, 290, T],            # goes back
               [1, 300, 316, T],            # does not start at 0
               [0, 299, 315, T - 1],        # does not end at total_q
               [0, 17, 316, T]):            # 299 new tokens for a sequence of 16
        out = torch.full_like(q, float("nan"))
        st = dbg.bi_attn_prefill(ctypes.byref(c.shape), _p(q), _p(k), _p(v),
                                 _p(torch.tensor(cu, dtype=torch.int32, device=dev())), _p(kvl),
                                 _p(bt), _p(c.kc), _p(c.vc), _p(out), None, T, max(c.pre),
                                 _stream())
        torch.cuda.synchronize()
        assert st == SHAPE_ERR and torch.isnan(out.float()).all(), cu
