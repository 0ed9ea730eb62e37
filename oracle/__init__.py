"""fp64 CPU oracle for batch-invariant RMSNorm, matmul and causal GQA attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
path (``invariant_bi_matmul_amd``) never imports, loads or calls it, and it
never imports the product path: the two share no code.

The arithmetic lives in ``bi_oracle.c`` (plain sequential fp64 loops; see its
header for the passages followed).  This module only builds that file with gcc,
marshals numpy arrays into it, and offers the results as float64 arrays.

Definitions (the pages name the three operations in the approach table of
"Defeating Nondeterminism in LLM Inference" as summarised on
mobiles-han.blogspot.com, and define none of them; these are the textbook
forms):

* ``rmsnorm``:   r = 1/sqrt(mean(x^2) + eps), y = x * r * gamma
* ``matmul``:    C = A @ W with W stored [K, N]
* ``attention``: causal softmax(scale * q.k) @ V at absolute positions, kv head
  of q head h = h // (n_q // n_kv); also returns lse = max z + ln(sum e^(z-max))

Pins that tie these to something other than themselves are in
``tests/test_oracle_*.py``.  Parity unpinned: nothing here is unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bi_oracle.c")
_LIB = os.path.join(_HERE, "libbi_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``bi_oracle.c`` into ``libbi_oracle.so`` (gcc, no fast-math)."""
    global _lib
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-pthread", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    _lib = None
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i64, i32, f64 = ctypes.c_int64, ctypes.c_int, ctypes.c_double
    lib.bio_abi_version.restype = i32
    lib.bio_bf16_decode.argtypes = [P, P, i64]
    lib.bio_bf16_encode.argtypes = [P, P, i64]
    lib.bio_rmsnorm_f64.argtypes = [P, P, i64, i64, f64, P, P, i32]
    lib.bio_matmul_f64.argtypes = [P, P, i64, i64, i64, P, i64, P, i32]
    lib.bio_matmul_f64.restype = i32
    lib.bio_attention_f64.argtypes = [P, P, P, P, P, P, i64, i32, i32, i32, f64, i32, P, P, i32]
    lib.bio_attention_f64.restype = i32
    _lib = lib
    return lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("oracle inputs are bf16 bit patterns (numpy uint16), got %s" % a.dtype)
    return a


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def bf16_decode(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64 (the oracle's own codec)."""
    b = _u16(bits)
    out = np.empty(b.shape, dtype=np.float64)
    _load().bio_bf16_decode(_ptr(b), _ptr(out), b.size)
    return out


def bf16_encode(x) -> np.ndarray:
    """bf16 bit patterns (uint16) of the nearest bf16 to each float64 value,
    rounded once, ties to even (the oracle's own codec)."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(a.shape, dtype=np.uint16)
    _load().bio_bf16_encode(_ptr(a), _ptr(out), a.size)
    return out


def rmsnorm(x_bits, gamma_bits, eps: float, threads: Optional[int] = None):
    """Returns (y [rows, H] float64, rstd [rows] float64)."""
    x = _u16(x_bits)
    g = _u16(gamma_bits)
    rows, hidden = x.shape
    if g.shape != (hidden,):
        raise ValueError("gamma must be [hidden]")
    y = np.empty((rows, hidden), dtype=np.float64)
    r = np.empty((rows,), dtype=np.float64)
    _load().bio_rmsnorm_f64(_ptr(x), _ptr(g), rows, hidden, float(eps), _ptr(y), _ptr(r),
                            threads or default_threads())
    return y, r


def matmul(a_bits, w_bits, rows: Optional[Sequence[int]] = None, threads: Optional[int] = None):
    """C = A @ W in fp64 with sequential k.  ``rows`` selects rows of A (C has
    len(rows) rows); default is every row."""
    a = _u16(a_bits)
    w = _u16(w_bits)
    m, k = a.shape
    k2, n = w.shape
    if k != k2:
        raise ValueError("inner dimensions differ")
    if rows is None:
        ridx = None
        nrows = m
    else:
        ridx = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        if ridx.size and (ridx.min() < 0 or ridx.max() >= m):
            raise IndexError("row index out of range")
        nrows = ridx.size
    c = np.empty((nrows, n), dtype=np.float64)
    rc = _load().bio_matmul_f64(_ptr(a), _ptr(w), m, n, k, _ptr(ridx), nrows, _ptr(c),
                                threads or default_threads())
    if rc:
        raise MemoryError("oracle matmul could not allocate")
    return c


def attention(q_bits, k_bits, v_bits, kv_lens: Sequence[int], tok_seq: Sequence[int],
              tok_pos: Sequence[int], scale: float, split: int = 0,
              threads: Optional[int] = None):
    """Causal GQA attention over logical keys/values.

    q_bits: [T, n_q, d]; k_bits, v_bits: [sum(kv_lens), n_kv, d], sequence b's
    rows back to back (row j of a sequence = absolute position j).  Query t
    belongs to sequence tok_seq[t] at position tok_pos[t] (< kv_lens[b]).
    split=0 evaluates the direct definition; split=S>0 evaluates partials over
    blocks [S*s, S*s+S) folded left in ascending s.
    Returns (out [T, n_q, d] float64, lse [T, n_q] float64, natural log).
    """
    q = _u16(q_bits)
    k = _u16(k_bits)
    v = _u16(v_bits)
    T, nq, d = q.shape
    _, nkv, d2 = k.shape
    if d2 != d or v.shape != k.shape:
        raise ValueError("k/v shape mismatch")
    lens = np.asarray(kv_lens, dtype=np.int64)
    off = np.zeros(len(lens) + 1, dtype=np.int64)
    off[1:] = np.cumsum(lens)
    if off[-1] != k.shape[0]:
        raise ValueError("sum(kv_lens) must equal the number of key rows")
    ts = np.ascontiguousarray(np.asarray(tok_seq, dtype=np.int32))
    tp = np.ascontiguousarray(np.asarray(tok_pos, dtype=np.int32))
    if ts.shape != (T,) or tp.shape != (T,):
        raise ValueError("tok_seq/tok_pos must have one entry per query")
    if T and (ts.min() < 0 or ts.max() >= len(lens)):
        raise IndexError("tok_seq out of range")
    if T and (tp.min() < 0 or np.any(tp >= lens[ts])):
        raise IndexError("tok_pos beyond the sequence's keys")
    out = np.empty((T, nq, d), dtype=np.float64)
    lse = np.empty((T, nq), dtype=np.float64)
    rc = _load().bio_attention_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(off), _ptr(ts), _ptr(tp), T,
                                   nq, nkv, d, float(scale), int(split), _ptr(out), _ptr(lse),
                                   threads or default_threads())
    if rc:
        raise ValueError("n_q must be a positive multiple of n_kv")
    return out, lse
