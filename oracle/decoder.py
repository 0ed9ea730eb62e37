"""fp64 oracle for the element-wise operations of a Llama-style decoder stack.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle``: only the test suite may
import it; the product path never does, and this module imports nothing from
the product path.

The pages define none of these operations (the news.hada.io page on GPT-4's
output varying at temperature 0 only states, in its problem statement, that
greedy decoding of a dense decoder is a function of the input and the
weights).  These are the textbook Llama forms, evaluated in float64 with no
intermediate rounding:

* ``embed``:   row gather, ids clamped into [0, vocab)
* ``rope``:    "rotate half" rotary embedding: for pair (i, i + d/2) with
  angle = pos * theta^(-2i/d): (a cos - b sin, a sin + b cos)
* ``swiglu``:  silu(g) * u with silu(g) = g / (1 + e^-g)
* ``add``:     a + b
* ``argmax``:  the first index of the largest value; NaN never chosen; a row
  with no number gives 0

Inputs that are bf16 arrive as bit patterns (numpy uint16) and are widened
exactly with the oracle's own codec.  Pins: ``tests/test_oracle_decoder.py``
(group property and closed forms of the rotation, closed forms of SiLU, tie
and NaN rules of argmax).  Parity unpinned: nothing here is unpinned.
"""
from __future__ import annotations

import numpy as np

from . import bf16_decode


def _f64(x) -> np.ndarray:
    x = np.asarray(x)
    return bf16_decode(x) if x.dtype == np.uint16 else x.astype(np.float64)


def embed(ids, table_bits) -> np.ndarray:
    """[T, H] float64 rows of the table, ids clamped into range."""
    table = bf16_decode(table_bits)
    ids = np.clip(np.asarray(ids, dtype=np.int64), 0, table.shape[0] - 1)
    return table[ids]


def rope(x, pos, theta: float) -> np.ndarray:
    """x [T, heads, d] (bf16 bits or float), pos [T] -> float64 [T, heads, d]."""
    x = _f64(x)
    d = x.shape[-1]
    half = d // 2
    i = np.arange(half, dtype=np.float64)
    inv_freq = float(theta) ** (-(2.0 * i) / d)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]  # [T, half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def silu(g) -> np.ndarray:
    g = _f64(g)
    return g / (1.0 + np.exp(-g))


def swiglu(gate, up) -> np.ndarray:
    return silu(gate) * _f64(up)


def add(a, b) -> np.ndarray:
    return _f64(a) + _f64(b)


def argmax(x) -> np.ndarray:
    """int64 [rows]: first index of the row maximum; NaN never chosen (NaN is
    read as -inf, and numpy's argmax returns the first maximal index)."""
    x = np.asarray(x, dtype=np.float64)
    return np.argmax(np.where(np.isnan(x), -np.inf, x), axis=1).astype(np.int64)
