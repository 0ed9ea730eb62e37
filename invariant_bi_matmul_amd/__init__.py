"""Batch-invariant RMSNorm, matmul and paged split-KV attention for MI355X.

A thin ctypes binding over ``libbi.so`` (built from ``csrc/`` by ``_build.py``;
the C interface and its contract are in ``include/bi.h``).  Every function
here only checks and marshals arguments -- dtype, shape, contiguity, device --
and hands raw device pointers plus torch's current HIP stream to the library.
All arithmetic runs in the library's HIP kernels; torch is used only to hold
device memory and streams.  If ``libbi.so`` is missing or cannot be loaded,
every call raises: there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "BIError", "lib_path", "debug_lib_path", "load", "load_library", "abi_version", "rmsnorm",
    "matmul", "matmul_pack_w", "matmul_packed", "attn_workspace_bytes",
    "attn_prefill", "attn_decode", "attn_decode_noalloc", "DECODE_SCRATCH_BYTES", "AttnShape",
    "SPLIT", "PAGE",
    "bix_rmsnorm_splitrow", "matmul_tile", "bix_matmul_splitk",
    "bix_attn_decode_splitkv",
    "embed", "rope", "swiglu", "add", "argmax", "matmul_ec_pack_w", "matmul_ec",
    "qkv_rope", "swiglu_pair",
    "attn_prefill_i16", "attn_decode_i16", "bix_mfma_loop",
    "bix_read_stream",
]

SPLIT = 256
PAGE = 16
DECODE_SCRATCH_BYTES = 64 << 20  # BI_DECODE_SCRATCH_BYTES
DTYPE_BF16, DTYPE_F32 = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


class BIError(RuntimeError):
    """A libbi call returned a non-OK status."""

    def __init__(self, fn: str, status: int, text: str):
        super().__init__("%s failed: status %d (%s)" % (fn, status, text))
        self.status = status


class AttnShape(ctypes.Structure):
    """Mirror of ``bi_attn_shape``."""
    _fields_ = [
        ("num_seqs", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
        ("num_pages", ctypes.c_int64), ("softmax_scale", ctypes.c_float),
    ]


def lib_path() -> str:
    return os.environ.get("BI_LIB", os.path.join(_HERE, "libbi.so"))


def load():
    """Load libbi.so (once).  Raises if it is absent: there is no fallback."""
    global _lib
    if _lib is None:
        _lib = load_library(lib_path())
    return _lib


def debug_lib_path() -> str:
    """The same library built with BI_DEBUG_CHECKS: its attention calls check
    kv_len, cu_q and the block table on the device before they launch, and
    return BI_ERR_INVALID_SHAPE for a bad entry (they synchronise the
    stream to do so).  Select it with BI_LIB=<this path>."""
    return os.path.join(_HERE, "libbi_debug.so")


def load_library(path: str):
    """A ctypes handle on the library at `path` with every signature set."""
    if not os.path.exists(path):
        raise RuntimeError("libbi.so not found at %s; build it with "
                           "`python -m invariant_bi_matmul_amd._build`" % path)
    lib = ctypes.CDLL(path)
    P, i64, i32, f32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float,
                            ctypes.c_size_t)
    SP = ctypes.POINTER(AttnShape)
    sigs = {
        "bi_abi_version": (ctypes.c_int, []),
        "bi_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "bi_rmsnorm": (ctypes.c_int, [P, P, P, P, i64, i64, f32, P]),
        "bi_matmul": (ctypes.c_int, [P, P, P, ctypes.c_int, i64, i64, i64, P]),
        "bi_matmul_packed": (ctypes.c_int, [P, P, P, ctypes.c_int, i64, i64, i64, P]),
        "bi_matmul_pack_w": (ctypes.c_int, [P, P, i64, i64, P]),
        "bix_matmul_splitk_packed": (ctypes.c_int, [P, P, P, ctypes.c_int, i64, i64, i64,
                                                    ctypes.c_int32, P, ctypes.c_size_t, P]),
        "bi_attn_workspace_bytes": (sz, [SP, i64, i32]),
        "bi_attn_prefill": (ctypes.c_int, [SP, P, P, P, P, P, P, P, P, P, P, i64, i32, P]),
        "bi_attn_decode": (ctypes.c_int, [SP, P, P, P, P, P, P, P, P, P, i32, P, sz, P]),
        "bi_attn_decode_noalloc": (ctypes.c_int, [SP, P, P, P, P, P, P, P, P, P, i32, P]),
        "bix_rmsnorm_splitrow": (ctypes.c_int, [P, P, P, P, i64, i64, f32, i32, P, sz, P]),
        "bix_matmul_tile": (ctypes.c_int, [i64, i64, P, P, P]),
        "bix_matmul_workspace_bytes": (sz, [i64, i64, i64, i32]),
        "bix_matmul_splitk": (ctypes.c_int, [P, P, P, ctypes.c_int, i64, i64, i64, i32, P, sz, P]),
        "bix_attn_decode_workspace_bytes": (sz, [SP, i32, i32]),
        "bix_attn_decode_splitkv": (ctypes.c_int,
                                    [SP, P, P, P, P, P, P, P, P, P, i32, i32, P, sz, P]),
        "bi_embed": (ctypes.c_int, [P, P, P, i64, i64, i64, P]),
        "bi_rope": (ctypes.c_int, [P, P, P, i64, i32, i32, i32, f32, P]),
        "bi_swiglu": (ctypes.c_int, [P, P, P, i64, P]),
        "bi_qkv_rope": (ctypes.c_int, [P, P, P, P, P, i64, i32, i32, i32, f32, P]),
        "bi_swiglu_pair": (ctypes.c_int, [P, P, i64, i64, P]),
        "bi_add": (ctypes.c_int, [P, P, P, i64, P]),
        "bi_argmax": (ctypes.c_int, [P, P, i64, i64, P]),
        "bix_mfma_loop": (ctypes.c_int, [i64, i32, i32, P, P]),
        "bix_read_stream": (ctypes.c_int, [P, i64, i32, P, P]),
        "bi_attn_prefill_i16": (ctypes.c_int,
                                [SP, P, P, P, P, P, P, P, P, P, P, P, P, i64, i32, P]),
        "bi_attn_decode_i16": (ctypes.c_int,
                               [SP, P, P, P, P, P, P, P, P, P, P, P, i32, P, sz, P]),
        "bi_matmul_ec_pack_w": (ctypes.c_int, [P, P, i64, i64, P]),
        "bi_matmul_ec_workspace_bytes": (sz, [i64, i64]),
        "bi_matmul_ec": (ctypes.c_int, [P, ctypes.c_int, P, P, ctypes.c_int, i64, i64, i64, P,
                                        sz, P]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def abi_version() -> int:
    return load().bi_abi_version()


def status_string(status: int) -> str:
    return load().bi_status_string(status).decode()


def _check(fn: str, status: int):
    if status != 0:
        raise BIError(fn, status, status_string(status))


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on the GPU" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    return t


# --------------------------------------------------------------------------- RMSNorm

def rmsnorm(x: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-6,
            out: Optional[torch.Tensor] = None, rstd: Optional[torch.Tensor] = None,
            with_rstd: bool = False):
    """y = bf16((x * rstd) * gamma), rstd = 1/sqrt(mean(x^2) + eps), per row.

    x: bf16 [rows, hidden]; gamma: bf16 [hidden].  ``out`` may be ``x``.
    Returns y, or (y, rstd) when ``with_rstd`` or ``rstd`` is given."""
    _dev(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be [rows, hidden]")
    rows, hidden = x.shape
    _dev(gamma, "gamma", torch.bfloat16, (hidden,))
    y = torch.empty_like(x) if out is None else _dev(out, "out", torch.bfloat16, x.shape)
    if rstd is None and with_rstd:
        rstd = torch.empty(rows, dtype=torch.float32, device=x.device)
    if rstd is not None:
        _dev(rstd, "rstd", torch.float32, (rows,))
    _check("bi_rmsnorm", load().bi_rmsnorm(_ptr(x), _ptr(gamma), _ptr(y), _ptr(rstd), rows, hidden,
                                           float(eps), _stream()))
    return (y, rstd) if rstd is not None else y


def bix_rmsnorm_splitrow(x, gamma, eps=1e-6, chunks: int = 0, out=None, rstd=None,
                         workspace=None):
    """Non-invariant comparator: each row's reduction split over ``chunks``
    workgroups (0 = chosen from the row count)."""
    _dev(x, "x", torch.bfloat16)
    rows, hidden = x.shape
    _dev(gamma, "gamma", torch.bfloat16, (hidden,))
    y = torch.empty_like(x) if out is None else _dev(out, "out", torch.bfloat16, x.shape)
    if rstd is not None:
        _dev(rstd, "rstd", torch.float32, (rows,))
    if workspace is None:
        workspace = torch.empty(max(rows, 1) * 64, dtype=torch.float32, device=x.device)
    _check("bix_rmsnorm_splitrow", load().bix_rmsnorm_splitrow(
        _ptr(x), _ptr(gamma), _ptr(y), _ptr(rstd), rows, hidden, float(eps), int(chunks),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream()))
    return (y, rstd) if rstd is not None else y


# --------------------------------------------------------------------------- matmul

def matmul(a: torch.Tensor, w: torch.Tensor, out: Optional[torch.Tensor] = None,
           out_dtype: torch.dtype = torch.bfloat16):
    """C = A @ W; a bf16 [m, k], w bf16 [k, n] (n contiguous); C bf16 or fp32."""
    _dev(a, "a", torch.bfloat16)
    _dev(w, "w", torch.bfloat16)
    if a.dim() != 2 or w.dim() != 2 or a.shape[1] != w.shape[0]:
        raise ValueError("need a [m, k] and w [k, n]")
    m, k = a.shape
    n = w.shape[1]
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out_dtype must be bfloat16 or float32")
    c = torch.empty(m, n, dtype=out_dtype, device=a.device) if out is None else \
        _dev(out, "out", out_dtype, (m, n))
    code = DTYPE_F32 if out_dtype == torch.float32 else DTYPE_BF16
    _check("bi_matmul", load().bi_matmul(_ptr(a), _ptr(w), _ptr(c), code, m, n, k, _stream()))
    return c


def matmul_pack_w(w: torch.Tensor, out: Optional[torch.Tensor] = None):
    """w bf16 [k, n] -> the strip layout bf16 [n/32, k, 32] (bi_matmul_pack_w)."""
    _dev(w, "w", torch.bfloat16)
    if w.dim() != 2:
        raise ValueError("need w [k, n]")
    k, n = w.shape
    if n % 32 != 0:
        raise ValueError("n must be a multiple of 32")
    wp = torch.empty(n // 32, k, 32, dtype=torch.bfloat16, device=w.device) if out is None else \
        _dev(out, "out", torch.bfloat16, (n // 32, k, 32))
    _check("bi_matmul_pack_w", load().bi_matmul_pack_w(_ptr(w), _ptr(wp), k, n, _stream()))
    return wp


def matmul_packed(a: torch.Tensor, wp: torch.Tensor, out: Optional[torch.Tensor] = None,
                  out_dtype: torch.dtype = torch.bfloat16):
    """C = A @ W with W given as matmul_pack_w(W) ([n/32, k, 32]); bitwise
    equal to matmul(a, W)."""
    _dev(a, "a", torch.bfloat16)
    _dev(wp, "wp", torch.bfloat16)
    if a.dim() != 2 or wp.dim() != 3 or wp.shape[2] != 32 or a.shape[1] != wp.shape[1]:
        raise ValueError("need a [m, k] and wp [n/32, k, 32]")
    m, k = a.shape
    n = wp.shape[0] * 32
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out_dtype must be bfloat16 or float32")
    c = torch.empty(m, n, dtype=out_dtype, device=a.device) if out is None else \
        _dev(out, "out", out_dtype, (m, n))
    code = DTYPE_F32 if out_dtype == torch.float32 else DTYPE_BF16
    _check("bi_matmul_packed", load().bi_matmul_packed(_ptr(a), _ptr(wp), _ptr(c), code, m, n, k,
                                                       _stream()))
    return c


def matmul_tile(m: int, n: int):
    """(tile_m, tile_n, workgroups) of bi_matmul for an m x n product on the
    current device (bix_matmul_tile; host-only, launches nothing)."""
    tm, tn, wg = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
    _check("bix_matmul_tile", load().bix_matmul_tile(int(m), int(n), ctypes.byref(tm),
                                                     ctypes.byref(tn), ctypes.byref(wg)))
    return tm.value, tn.value, wg.value


def bix_matmul_splitk(a, w, split_k: int = 0, out=None, out_dtype=torch.bfloat16,
                      workspace=None):
    """Non-invariant comparator: split-K with ``split_k`` slices (0 = chosen
    from the grid size).  A 3-D ``w`` is taken as matmul_pack_w's strip layout
    [n/32, k, 32] (bix_matmul_splitk_packed)."""
    _dev(a, "a", torch.bfloat16)
    _dev(w, "w", torch.bfloat16)
    m, k = a.shape
    packed = w.dim() == 3
    n = w.shape[0] * 32 if packed else w.shape[1]
    c = torch.empty(m, n, dtype=out_dtype, device=a.device) if out is None else \
        _dev(out, "out", out_dtype, (m, n))
    lib = load()
    need = lib.bix_matmul_workspace_bytes(m, n, k, int(split_k))
    if workspace is None:
        workspace = torch.empty(max(need, 16) // 4 + 4, dtype=torch.float32, device=a.device)
    code = DTYPE_F32 if out_dtype == torch.float32 else DTYPE_BF16
    fn = lib.bix_matmul_splitk_packed if packed else lib.bix_matmul_splitk
    _check("bix_matmul_splitk", fn(
        _ptr(a), _ptr(w), _ptr(c), code, m, n, k, int(split_k), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream()))
    return c


# --------------------------------------------------------------------------- attention

def make_shape(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
               max_pages_per_seq: int, num_pages: int, softmax_scale: float) -> AttnShape:
    return AttnShape(num_seqs, num_q_heads, num_kv_heads, head_dim, PAGE, max_pages_per_seq,
                     num_pages, softmax_scale)


def _cache_shape(k_cache: torch.Tensor, v_cache: torch.Tensor):
    _dev(k_cache, "k_cache", torch.bfloat16)
    _dev(v_cache, "v_cache", torch.bfloat16, k_cache.shape)
    if k_cache.dim() != 4 or k_cache.shape[2] != PAGE:
        raise ValueError("caches must be [num_pages, n_kv, 16, d]")
    return k_cache.shape


def attn_workspace_bytes(shape: AttnShape, num_tokens: int, max_kv_len: int) -> int:
    return int(load().bi_attn_workspace_bytes(ctypes.byref(shape), num_tokens, max_kv_len))


def attn_prefill(q, k_new, v_new, cu_q, kv_len, block_table, k_cache, v_cache, softmax_scale,
                 max_q_per_seq: int, out=None, lse=None, with_lse: bool = False):
    """Append k_new/v_new to the paged caches, then causal attention for q.

    q bf16 [T, n_q, d]; k_new/v_new bf16 [T, n_kv, d]; cu_q int32 [B+1];
    kv_len int32 [B] (after the append); block_table int32 [B, max_pages];
    caches bf16 [P, n_kv, 16, d].  Returns out (and lse)."""
    P, nkv, _, d = _cache_shape(k_cache, v_cache)
    _dev(q, "q", torch.bfloat16)
    T, nq, dq = q.shape
    if dq != d:
        raise ValueError("head_dim mismatch")
    _dev(k_new, "k_new", torch.bfloat16, (T, nkv, d))
    _dev(v_new, "v_new", torch.bfloat16, (T, nkv, d))
    _dev(block_table, "block_table", torch.int32)
    B, maxp = block_table.shape
    _dev(cu_q, "cu_q", torch.int32, (B + 1,))
    _dev(kv_len, "kv_len", torch.int32, (B,))
    o = torch.empty_like(q) if out is None else _dev(out, "out", torch.bfloat16, q.shape)
    if lse is None and with_lse:
        lse = torch.empty(T, nq, dtype=torch.float32, device=q.device)
    if lse is not None:
        _dev(lse, "lse", torch.float32, (T, nq))
    shape = make_shape(B, nq, nkv, d, maxp, P, softmax_scale)
    _check("bi_attn_prefill", load().bi_attn_prefill(
        ctypes.byref(shape), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(cu_q), _ptr(kv_len),
        _ptr(block_table), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse), T,
        int(max_q_per_seq), _stream()))
    return (o, lse) if lse is not None else o


def _decode_args(q, k_new, v_new, kv_len, block_table, k_cache, v_cache, out, lse, with_lse):
    P, nkv, _, d = _cache_shape(k_cache, v_cache)
    _dev(q, "q", torch.bfloat16)
    B, nq, dq = q.shape
    if dq != d:
        raise ValueError("head_dim mismatch")
    _dev(k_new, "k_new", torch.bfloat16, (B, nkv, d))
    _dev(v_new, "v_new", torch.bfloat16, (B, nkv, d))
    _dev(block_table, "block_table", torch.int32)
    if block_table.shape[0] != B:
        raise ValueError("block_table needs one row per sequence")
    _dev(kv_len, "kv_len", torch.int32, (B,))
    o = torch.empty_like(q) if out is None else _dev(out, "out", torch.bfloat16, q.shape)
    if lse is None and with_lse:
        lse = torch.empty(B, nq, dtype=torch.float32, device=q.device)
    if lse is not None:
        _dev(lse, "lse", torch.float32, (B, nq))
    return B, nq, nkv, d, P, block_table.shape[1], o, lse


def attn_decode(q, k_new, v_new, kv_len, block_table, k_cache, v_cache, softmax_scale,
                max_kv_len: int, workspace=None, out=None, lse=None, with_lse: bool = False):
    """One new token per sequence: append, then split-parallel attention with a
    fixed-order combine.  q bf16 [B, n_q, d]; k_new/v_new bf16 [B, n_kv, d]."""
    B, nq, nkv, d, P, maxp, o, lse = _decode_args(q, k_new, v_new, kv_len, block_table, k_cache,
                                                  v_cache, out, lse, with_lse)
    shape = make_shape(B, nq, nkv, d, maxp, P, softmax_scale)
    lib = load()
    need = lib.bi_attn_workspace_bytes(ctypes.byref(shape), B, int(max_kv_len))
    if workspace is None:
        workspace = torch.empty(max(need, 16) // 4 + 4, dtype=torch.float32, device=q.device)
    _check("bi_attn_decode", lib.bi_attn_decode(
        ctypes.byref(shape), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(kv_len), _ptr(block_table),
        _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse), int(max_kv_len), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream()))
    return (o, lse) if lse is not None else o


def attn_decode_noalloc(q, k_new, v_new, kv_len, block_table, k_cache, v_cache, softmax_scale,
                        max_kv_len: int, out=None, lse=None, with_lse: bool = False):
    """attn_decode without a workspace: the library keeps the split partials in
    its own per-GPU scratch array (DECODE_SCRATCH_BYTES) and allocates nothing.
    Calls that may overlap on one GPU race on that array."""
    B, nq, nkv, d, P, maxp, o, lse = _decode_args(q, k_new, v_new, kv_len, block_table, k_cache,
                                                  v_cache, out, lse, with_lse)
    shape = make_shape(B, nq, nkv, d, maxp, P, softmax_scale)
    _check("bi_attn_decode_noalloc", load().bi_attn_decode_noalloc(
        ctypes.byref(shape), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(kv_len), _ptr(block_table),
        _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse), int(max_kv_len), _stream()))
    return (o, lse) if lse is not None else o


def bix_attn_decode_splitkv(q, k_new, v_new, kv_len, block_table, k_cache, v_cache,
                            softmax_scale, max_kv_len: int, num_splits: int = 0, workspace=None,
                            out=None, lse=None, with_lse: bool = False):
    """Non-invariant comparator: decode with a split count chosen from the
    batch (0 = the library's heuristic)."""
    B, nq, nkv, d, P, maxp, o, lse = _decode_args(q, k_new, v_new, kv_len, block_table, k_cache,
                                                  v_cache, out, lse, with_lse)
    shape = make_shape(B, nq, nkv, d, maxp, P, softmax_scale)
    lib = load()
    need = lib.bix_attn_decode_workspace_bytes(ctypes.byref(shape), int(max_kv_len),
                                               int(num_splits))
    if workspace is None:
        workspace = torch.empty(max(need, 16) // 4 + 4, dtype=torch.float32, device=q.device)
    _check("bix_attn_decode_splitkv", lib.bix_attn_decode_splitkv(
        ctypes.byref(shape), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(kv_len), _ptr(block_table),
        _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse), int(max_kv_len), int(num_splits),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream()))
    return (o, lse) if lse is not None else o


# --------------------------------------------------------------------------- decoder stack

def embed(ids: torch.Tensor, table: torch.Tensor, out: Optional[torch.Tensor] = None):
    """out[t] = table[ids[t]] (ids clamped into range); ids int32 [T], table bf16 [V, H]."""
    _dev(ids, "ids", torch.int32)
    _dev(table, "table", torch.bfloat16)
    if ids.dim() != 1 or table.dim() != 2:
        raise ValueError("need ids [T] and table [V, H]")
    T, (V, H) = ids.shape[0], table.shape
    o = torch.empty(T, H, dtype=torch.bfloat16, device=table.device) if out is None else \
        _dev(out, "out", torch.bfloat16, (T, H))
    _check("bi_embed", load().bi_embed(_ptr(ids), _ptr(table), _ptr(o), T, H, V, _stream()))
    return o


def rope(q: torch.Tensor, k: torch.Tensor, pos: torch.Tensor, theta: float):
    """Rotary embedding in place ("rotate half"); q bf16 [T, n_q, d], k bf16
    [T, n_kv, d], pos int32 [T].  Returns (q, k)."""
    _dev(q, "q", torch.bfloat16)
    _dev(k, "k", torch.bfloat16)
    if q.dim() != 3 or k.dim() != 3 or q.shape[0] != k.shape[0] or q.shape[2] != k.shape[2]:
        raise ValueError("need q [T, n_q, d] and k [T, n_kv, d]")
    T, nq, d = q.shape
    _dev(pos, "pos", torch.int32, (T,))
    _check("bi_rope", load().bi_rope(_ptr(q), _ptr(k), _ptr(pos), T, nq, k.shape[1], d,
                                     float(theta), _stream()))
    return q, k


def swiglu(gate: torch.Tensor, up: torch.Tensor, out: Optional[torch.Tensor] = None):
    """bf16(silu(gate) * up), same shape as gate."""
    _dev(gate, "gate", torch.bfloat16)
    _dev(up, "up", torch.bfloat16, gate.shape)
    o = torch.empty_like(gate) if out is None else _dev(out, "out", torch.bfloat16, gate.shape)
    _check("bi_swiglu", load().bi_swiglu(_ptr(gate), _ptr(up), _ptr(o), gate.numel(), _stream()))
    return o


def qkv_rope(qkv: torch.Tensor, pos: torch.Tensor, n_q: int, n_kv: int, theta: float,
             q: Optional[torch.Tensor] = None, k: Optional[torch.Tensor] = None,
             v: Optional[torch.Tensor] = None):
    """Split a fused q|k|v projection output qkv bf16 [T, (n_q + 2 n_kv) * d]
    into q [T, n_q, d], k and v [T, n_kv, d], rotating q and k as ``rope``
    does.  Returns (q, k, v)."""
    _dev(qkv, "qkv", torch.bfloat16)
    if qkv.dim() != 2 or qkv.shape[1] % (n_q + 2 * n_kv) != 0:
        raise ValueError("need qkv [T, (n_q + 2 n_kv) * d]")
    T = qkv.shape[0]
    d = qkv.shape[1] // (n_q + 2 * n_kv)
    _dev(pos, "pos", torch.int32, (T,))
    new = lambda t, h, name: (torch.empty(T, h, d, dtype=torch.bfloat16, device=qkv.device)
                              if t is None else _dev(t, name, torch.bfloat16, (T, h, d)))
    q, k, v = new(q, n_q, "q"), new(k, n_kv, "k"), new(v, n_kv, "v")
    _check("bi_qkv_rope", load().bi_qkv_rope(_ptr(qkv), _ptr(pos), _ptr(q), _ptr(k), _ptr(v), T,
                                             n_q, n_kv, d, float(theta), _stream()))
    return q, k, v


def swiglu_pair(gu: torch.Tensor, out: Optional[torch.Tensor] = None):
    """``swiglu`` over a fused gate|up projection output gu bf16 [rows, 2f]
    (gate columns first); returns bf16 [rows, f]."""
    _dev(gu, "gu", torch.bfloat16)
    if gu.dim() != 2 or gu.shape[1] % 2 != 0:
        raise ValueError("need gu [rows, 2f]")
    rows, f = gu.shape[0], gu.shape[1] // 2
    o = (torch.empty(rows, f, dtype=torch.bfloat16, device=gu.device) if out is None
         else _dev(out, "out", torch.bfloat16, (rows, f)))
    _check("bi_swiglu_pair", load().bi_swiglu_pair(_ptr(gu), _ptr(o), rows, f, _stream()))
    return o


def add(a: torch.Tensor, b: torch.Tensor, out: Optional[torch.Tensor] = None):
    """bf16(a + b); ``out`` may be ``a``."""
    _dev(a, "a", torch.bfloat16)
    _dev(b, "b", torch.bfloat16, a.shape)
    o = torch.empty_like(a) if out is None else _dev(out, "out", torch.bfloat16, a.shape)
    _check("bi_add", load().bi_add(_ptr(a), _ptr(b), _ptr(o), a.numel(), _stream()))
    return o


def argmax(x: torch.Tensor, out: Optional[torch.Tensor] = None):
    """Row-wise argmax of fp32 [rows, n] (lowest index on ties); int32 [rows]."""
    _dev(x, "x", torch.float32)
    if x.dim() != 2:
        raise ValueError("x must be [rows, n]")
    rows, n = x.shape
    o = torch.empty(rows, dtype=torch.int32, device=x.device) if out is None else \
        _dev(out, "out", torch.int32, (rows,))
    _check("bi_argmax", load().bi_argmax(_ptr(x), _ptr(o), rows, n, _stream()))
    return o


# --------------------------------------------------------------------------- error-compensated matmul

def matmul_ec_pack_w(w: torch.Tensor, out: Optional[torch.Tensor] = None):
    """Pack an fp32 weight [k, n] as bf16 [3k, n] = [hi; lo; hi] for ``matmul_ec``."""
    _dev(w, "w", torch.float32)
    if w.dim() != 2:
        raise ValueError("w must be [k, n]")
    k, n = w.shape
    o = torch.empty(3 * k, n, dtype=torch.bfloat16, device=w.device) if out is None else \
        _dev(out, "out", torch.bfloat16, (3 * k, n))
    _check("bi_matmul_ec_pack_w", load().bi_matmul_ec_pack_w(_ptr(w), _ptr(o), k, n, _stream()))
    return o


def matmul_ec(a: torch.Tensor, w3: torch.Tensor, out: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None, out_dtype=torch.float32):
    """C = hi(a)hi(w) + hi(a)lo(w) + lo(a)hi(w) for a [m, k] (fp32, or bf16,
    whose lo is 0 and whose third product is skipped) and a weight packed by
    ``matmul_ec_pack_w`` (bf16 [3k, n]); C fp32 or its bf16 rounding."""
    if not isinstance(a, torch.Tensor) or a.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("a must be a float32 or bfloat16 tensor")
    _dev(a, "a", a.dtype)
    _dev(w3, "w3", torch.bfloat16)
    if a.dim() != 2 or w3.dim() != 2 or w3.shape[0] != 3 * a.shape[1]:
        raise ValueError("need a [m, k] and w3 [3k, n]")
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be float32 or bfloat16")
    m, k = a.shape
    n = w3.shape[1]
    c = torch.empty(m, n, dtype=out_dtype, device=a.device) if out is None else \
        _dev(out, "out", out_dtype, (m, n))
    lib = load()
    need = lib.bi_matmul_ec_workspace_bytes(m, k)
    if workspace is None:
        workspace = torch.empty(max(need, 16) // 2 + 8, dtype=torch.bfloat16, device=a.device)
    a_dt = DTYPE_F32 if a.dtype == torch.float32 else DTYPE_BF16
    c_dt = DTYPE_F32 if out_dtype == torch.float32 else DTYPE_BF16
    _check("bi_matmul_ec", lib.bi_matmul_ec(_ptr(a), a_dt, _ptr(w3), _ptr(c), c_dt, m, n, k,
                                            _ptr(workspace),
                                            workspace.numel() * workspace.element_size(),
                                            _stream()))
    return c


# --------------------------------------------------------------------------- int16 KV cache

def _i16_cache(k_cache, v_cache, k_scale, v_scale):
    _dev(k_cache, "k_cache", torch.int16)
    _dev(v_cache, "v_cache", torch.int16, k_cache.shape)
    if k_cache.dim() != 4 or k_cache.shape[2] != PAGE:
        raise ValueError("caches must be int16 [num_pages, n_kv, 16, d]")
    P, nkv, _, d = k_cache.shape
    _dev(k_scale, "k_scale", torch.float32, (P, nkv, PAGE))
    _dev(v_scale, "v_scale", torch.float32, (P, nkv, PAGE))
    return P, nkv, d


def attn_prefill_i16(q, k_new, v_new, cu_q, kv_len, block_table, k_cache, v_cache, k_scale,
                     v_scale, softmax_scale, max_q_per_seq: int, out=None, lse=None,
                     with_lse: bool = False):
    """``attn_prefill`` over the int16 cache: k_new/v_new (bf16) are quantised
    per (token, kv head) into k_cache/v_cache (int16 [P, n_kv, 16, d]) with
    their factors in k_scale/v_scale (fp32 [P, n_kv, 16])."""
    P, nkv, d = _i16_cache(k_cache, v_cache, k_scale, v_scale)
    _dev(q, "q", torch.bfloat16)
    T, nq, dq = q.shape
    if dq != d:
        raise ValueError("head_dim mismatch")
    _dev(k_new, "k_new", torch.bfloat16, (T, nkv, d))
    _dev(v_new, "v_new", torch.bfloat16, (T, nkv, d))
    _dev(block_table, "block_table", torch.int32)
    B, maxp = block_table.shape
    _dev(cu_q, "cu_q", torch.int32, (B + 1,))
    _dev(kv_len, "kv_len", torch.int32, (B,))
    o = torch.empty_like(q) if out is None else _dev(out, "out", torch.bfloat16, q.shape)
    if lse is None and with_lse:
        lse = torch.empty(T, nq, dtype=torch.float32, device=q.device)
    if lse is not None:
        _dev(lse, "lse", torch.float32, (T, nq))
    shape = make_shape(B, nq, nkv, d, maxp, P, softmax_scale)
    _check("bi_attn_prefill_i16", load().bi_attn_prefill_i16(
        ctypes.byref(shape), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(cu_q), _ptr(kv_len),
        _ptr(block_table), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(o),
        _ptr(lse), T, int(max_q_per_seq), _stream()))
    return (o, lse) if lse is not None else o


def attn_decode_i16(q, k_new, v_new, kv_len, block_table, k_cache, v_cache, k_scale, v_scale,
                    softmax_scale, max_kv_len: Optional[int] = None, workspace=None, out=None,
                    lse=None, with_lse: bool = False):
    """One new token per sequence over the int16 cache; q bf16 [B, n_q, d].
    ``max_kv_len`` (host) bounds every kv_len after the append; by default the
    block table's capacity."""
    P, nkv, d = _i16_cache(k_cache, v_cache, k_scale, v_scale)
    _dev(q, "q", torch.bfloat16)
    B, nq, dq = q.shape
    if dq != d:
        raise ValueError("head_dim mismatch")
    _dev(k_new, "k_new", torch.bfloat16, (B, nkv, d))
    _dev(v_new, "v_new", torch.bfloat16, (B, nkv, d))
    _dev(block_table, "block_table", torch.int32)
    if block_table.shape[0] != B:
        raise ValueError("block_table needs one row per sequence")
    _dev(kv_len, "kv_len", torch.int32, (B,))
    o = torch.empty_like(q) if out is None else _dev(out, "out", torch.bfloat16, q.shape)
    if lse is None and with_lse:
        lse = torch.empty(B, nq, dtype=torch.float32, device=q.device)
    if lse is not None:
        _dev(lse, "lse", torch.float32, (B, nq))
    shape = make_shape(B, nq, nkv, d, block_table.shape[1], P, softmax_scale)
    if max_kv_len is None:
        max_kv_len = block_table.shape[1] * PAGE
    need = attn_workspace_bytes(shape, B, max_kv_len)
    if workspace is None:
        workspace = torch.empty(max(need, 16) // 4 + 4, dtype=torch.float32, device=q.device)
    _check("bi_attn_decode_i16", load().bi_attn_decode_i16(
        ctypes.byref(shape), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(kv_len), _ptr(block_table),
        _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(o), _ptr(lse),
        int(max_kv_len), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream()))
    return (o, lse) if lse is not None else o


# --------------------------------------------------------------------------- measurement

def bix_mfma_loop(iters: int, workgroups: int, sink: Optional[torch.Tensor] = None,
                  varied: bool = False):
    """Measurement only: ``workgroups`` x 4 waves each run ``iters`` rounds of four
    independent bf16 32x32x16 MFMAs in registers (``varied``: on operands that
    change from one MFMA to the next).  Returns the flop count."""
    if sink is None:
        sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    _check("bix_mfma_loop", load().bix_mfma_loop(int(iters), int(workgroups), int(bool(varied)),
                                                 _ptr(sink), _stream()))
    return 4.0 * 4 * 32768 * iters * workgroups


def bix_read_stream(x: torch.Tensor, workgroups: int, sink: Optional[torch.Tensor] = None):
    """Measurement only: read every byte of the contiguous device tensor ``x``
    once.  Returns the byte count."""
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=x.device)
    nbytes = x.numel() * x.element_size()
    _check("bix_read_stream", load().bix_read_stream(_ptr(x), nbytes, int(workgroups), _ptr(sink),
                                                     _stream()))
    return nbytes
