"""The C-ABI library without a GPU: it loads, exports every function bi.h
declares, and rejects bad arguments with the documented status before any
HIP call (so these run on a host with no GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bi.h")

OK, NULLP, SHAPE, UNSUP, WS = 0, 1, 2, 3, 4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:bi|bix)_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import invariant_bi_matmul_amd as bi
    if not os.path.exists(bi.lib_path()):
        pytest.fail("libbi.so is not built (python -m invariant_bi_matmul_amd._build)")
    return bi.load()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert "bi_matmul" in names and "bi_attn_decode" in names and len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n


def test_debug_build_exports_the_same_functions():
    """libbi_debug.so (attention calls validate their device index arrays)
    is the same interface."""
    from invariant_bi_matmul_amd import _build
    if not os.path.exists(_build.DEBUG_LIB):
        pytest.fail("libbi_debug.so is not built (python -m invariant_bi_matmul_amd._build)")
    dbg = ctypes.CDLL(_build.DEBUG_LIB)
    for n in declared_functions():
        assert hasattr(dbg, n), n
    assert dbg.bi_abi_version() == 5


def test_version_and_status_strings(lib):
    assert lib.bi_abi_version() == 5
    for s in range(7):
        assert lib.bi_status_string(s)
    assert lib.bi_status_string(99) == b"unknown status"


def _p(v=0x1000):
    return ctypes.c_void_p(v)


def test_rmsnorm_validation(lib):
    f = lib.bi_rmsnorm
    assert f(_p(), _p(), _p(), None, -1, 4096, 1e-6, None) == SHAPE
    assert f(_p(), _p(), _p(), None, 4, 4100, 1e-6, None) == UNSUP
    assert f(_p(), _p(), _p(), None, 4, 32768, 1e-6, None) == UNSUP
    assert f(None, _p(), _p(), None, 4, 4096, 1e-6, None) == NULLP
    assert f(_p(0x1008), _p(), _p(), None, 4, 4096, 1e-6, None) == SHAPE
    assert f(_p(), _p(), _p(), None, 4, 4096, -1.0, None) == SHAPE
    assert f(None, None, None, None, 0, 4096, 1e-6, None) == OK  # empty: no-op
    assert lib.bix_rmsnorm_splitrow(_p(), _p(), _p(), None, 4, 4096, 1e-6, 2, _p(), 16,
                                    None) == WS


def test_matmul_validation(lib):
    f = lib.bi_matmul
    assert f(_p(), _p(), _p(), 0, 4, 4096, 100, None) == UNSUP      # k % 64
    assert f(_p(), _p(), _p(), 0, 4, 4100, 4096, None) == UNSUP     # n % 8
    assert f(_p(), _p(), _p(), 7, 4, 4096, 4096, None) == SHAPE     # dtype
    assert f(_p(), _p(), _p(), 0, -4, 4096, 4096, None) == SHAPE
    assert f(_p(), None, _p(), 0, 4, 4096, 4096, None) == NULLP
    assert f(None, None, None, 0, 0, 4096, 4096, None) == OK
    assert lib.bix_matmul_workspace_bytes(8, 4096, 4096, 4) == 4 * 8 * 4096 * 4
    assert lib.bix_matmul_splitk(_p(), _p(), _p(), 0, 8, 4096, 4096, 4, _p(), 1024, None) == WS


def test_matmul_packed_validation(lib):
    f = lib.bi_matmul_packed
    assert f(_p(), _p(), _p(), 0, 4, 4104, 4096, None) == UNSUP     # n % 32
    assert f(_p(), _p(), _p(), 0, 4, 4096, 100, None) == UNSUP      # k % 64
    assert f(_p(), _p(), _p(), 0, -4, 4096, 4096, None) == SHAPE
    assert f(_p(), None, _p(), 0, 4, 4096, 4096, None) == NULLP
    assert f(None, None, None, 0, 0, 4096, 4096, None) == OK
    g = lib.bi_matmul_pack_w
    assert g(_p(), _p(), 4096, 4104, None) == UNSUP                  # n % 32
    assert g(_p(), _p(), -1, 4096, None) == SHAPE
    assert g(None, _p(), 4096, 4096, None) == NULLP
    assert g(_p(0x1008), _p(), 4096, 4096, None) == SHAPE            # alignment
    assert g(None, None, 0, 4096, None) == OK                         # empty: no-op


def test_matmul_tile_choice(lib):
    """The tile bi_matmul picks (256 CUs, the MI355X count and the host-only
    fallback): the first of 64 x 32, 64 x 64, 128 x 64, 128 x 128 whose tiles fit one
    per CU; else, with several row-tiles, the persistent 256 x 256 tile where
    ceil(tiles / CUs) rounds at 1.6 times the time per tile beat those of the
    persistent 256 x 128 tile, else the latter."""
    import invariant_bi_matmul_amd as bi
    cases = {(1, 4096): (64, 32, 128), (128, 4096): (64, 32, 256), (129, 4096): (64, 64, 192),
             (1, 6144): (64, 32, 192), (1, 14336): (64, 64, 224),
             (256, 4096): (64, 64, 256), (257, 4096): (128, 64, 192),
             (512, 4096): (128, 64, 256), (513, 4096): (128, 128, 160),
             (1024, 4096): (128, 128, 256), (1025, 4096): (256, 128, 160),
             (2048, 4096): (256, 128, 256), (4096, 4096): (256, 256, 256),
             (1536, 14336): (256, 128, 256), (1537, 14336): (256, 256, 256),
             (2048, 14336): (256, 256, 256), (2048, 6144): (256, 256, 192),
             (64, 28672): (128, 128, 224), (1, 128256): (256, 128, 256),
             (256, 128256): (256, 128, 256), (300, 128256): (256, 256, 256),
             (5, 8): (64, 32, 1)}
    for (m, n), want in cases.items():
        assert bi.matmul_tile(m, n) == want, (m, n)
    assert lib.bix_matmul_tile(0, 4096, None, None, None) == SHAPE
    assert lib.bix_matmul_tile(8, 4096, None, None, None) == OK


def _shape(**kw):
    import invariant_bi_matmul_amd as bi
    base = dict(num_seqs=2, num_q_heads=32, num_kv_heads=8, head_dim=128, max_pages_per_seq=4,
                num_pages=8, softmax_scale=0.088388346)
    base.update(kw)
    s = bi.make_shape(**base)
    return s


def test_attention_validation(lib):
    import invariant_bi_matmul_amd as bi
    s = _shape()
    by = ctypes.byref
    assert lib.bi_attn_workspace_bytes(by(s), 2, 300) == 2 * 32 * 2 * 132 * 4
    assert lib.bi_attn_workspace_bytes(by(_shape(head_dim=96)), 2, 300) == 0
    args = [_p()] * 9 + [None]
    assert lib.bi_attn_prefill(by(_shape(head_dim=96)), *args, 10, 5, None) == UNSUP
    assert lib.bi_attn_prefill(by(_shape(num_kv_heads=5)), *args, 10, 5, None) == SHAPE
    assert lib.bi_attn_prefill(by(_shape(num_q_heads=64, num_kv_heads=2)), *args, 10, 5,
                               None) == UNSUP  # group 32 > 16
    bad_page = _shape()
    bad_page.page_size = 32
    assert lib.bi_attn_prefill(by(bad_page), *args, 10, 5, None) == UNSUP
    assert lib.bi_attn_prefill(by(s), *args, 10, 65, None) == SHAPE  # > 4 pages * 16
    assert lib.bi_attn_prefill(by(s), *([None] + [_p()] * 8 + [None]), 10, 5, None) == NULLP
    assert lib.bi_attn_prefill(by(s), *args, 0, 0, None) == OK
    dec = [_p()] * 8 + [None]
    assert lib.bi_attn_decode(by(s), *dec, 60, _p(), 16, None) == WS
    assert lib.bi_attn_decode(by(s), *dec, 65, _p(), 1 << 30, None) == SHAPE
    assert lib.bi_attn_decode(by(_shape(num_seqs=0)), *dec, 0, None, 0, None) == OK
    assert bi.SPLIT == 256 and bi.PAGE == 16


def test_decode_noalloc_validation(lib):
    """The no-allocation decode refuses, before any HIP call, a call whose
    split records would not fit its scratch array."""
    import invariant_bi_matmul_amd as bi
    by = ctypes.byref
    dec = [_p()] * 8 + [None]
    big = _shape(num_seqs=64, max_pages_per_seq=2048)
    assert lib.bi_attn_workspace_bytes(by(big), 64, 32768) > bi.DECODE_SCRATCH_BYTES
    assert lib.bi_attn_decode_noalloc(by(big), *dec, 32768, None) == WS
    assert lib.bi_attn_decode_noalloc(by(_shape()), *dec, 65, None) == SHAPE
    assert lib.bi_attn_decode_noalloc(by(_shape(head_dim=96)), *dec, 60, None) == UNSUP
    assert lib.bi_attn_decode_noalloc(by(_shape()), *([None] + [_p()] * 7 + [None]), 60,
                                      None) == NULLP
    assert lib.bi_attn_decode_noalloc(by(_shape(num_seqs=0)), *dec, 0, None) == OK
