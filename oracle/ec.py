"""fp64 oracle for the error-compensated matmul.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle``: only the test suite may
import it; it imports nothing from the product path.

The HEAL page on gist.science ("Demystifying Numerical Instability in LLM
Inference ... with HEAL"), item 2 of its new-solution section, splits a GEMM
into a main low-precision product and a clean-up product that recovers what
the main one dropped; it gives no formula.  The reading followed: each fp32
operand x is split into hi = bf16(x) and lo = bf16(x - hi) (round to nearest
even; a non-finite hi gets lo = 0), and

    C = hi(A) hi(W) + hi(A) lo(W) + lo(A) hi(W)          (lo lo dropped)

``split`` is that split, written with integer rounding on the fp32 bits (its
own code, not the GPU's conversion); ``ec_product`` evaluates the formula in
float64 (no accumulation error), ``exact`` is A W of the fp32 values in
float64.  Pins: ``tests/test_oracle_ec.py``.  Parity unpinned: nothing here is
unpinned.
"""
from __future__ import annotations

import numpy as np


def _round_bf16(x32: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), returned as fp32 values."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32).copy()
    nan = np.isnan(x32)
    out[nan] = x32[nan]
    return out


def split(x) -> tuple:
    """(hi, lo) of fp32 values, both bf16-representable, as float64 arrays."""
    x32 = np.asarray(x, dtype=np.float32)
    hi = _round_bf16(x32)
    with np.errstate(invalid="ignore", over="ignore"):
        rest = (x32 - hi).astype(np.float32)  # exact in fp32
    lo = np.where(np.isfinite(hi), _round_bf16(rest), np.float32(0.0))
    return hi.astype(np.float64), lo.astype(np.float64)


def ec_product(a, w) -> np.ndarray:
    """hi(a)hi(w) + hi(a)lo(w) + lo(a)hi(w) in float64."""
    ah, al = split(a)
    wh, wl = split(w)
    return ah @ wh + ah @ wl + al @ wh


def exact(a, w) -> np.ndarray:
    """A W of the fp32 values in float64."""
    return np.asarray(a, dtype=np.float32).astype(np.float64) @ \
        np.asarray(w, dtype=np.float32).astype(np.float64)
