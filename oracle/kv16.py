"""Oracle for the int16 KV cache: the quantiser and attention over the
dequantised keys and values.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle``: only the test suite may
import it; it imports nothing from the product path.

The HEAL page on gist.science ("Demystifying Numerical Instability in LLM
Inference ... with HEAL"), item 1 of its new-solution section, stores the
attention keys and values as INT16 and unpacks them exactly into two 16-bit
values for the matrix units.  The page gives no formula; the reading followed:

* ``quantize``: per (token, kv head) row x (bf16), s = max |x|, then
  q = rint(x * (32767 / s)) clipped to +-32767 (ties to even) and
  f = s / 32767, all in IEEE fp32 -- the kernel's precision, so that both
  sides take each integer decision the same way -- with q = 0, f = 0 for an
  all-zero row;
* ``attention``: causal GQA softmax attention in float64 over the
  dequantised values q * f (exact in float64), the direct definition.

Pins: ``tests/test_oracle_kv16.py``.  Parity unpinned: nothing here is
unpinned.
"""
from __future__ import annotations

import numpy as np

from . import bf16_decode


def quantize(x_bits):
    """x_bits: bf16 bit patterns [..., d] -> (q int16 [..., d], f float32 [...])."""
    x = bf16_decode(x_bits).astype(np.float32)          # exact widening
    s = np.max(np.abs(x), axis=-1)                       # fp32, exact
    with np.errstate(divide="ignore", invalid="ignore"):
        inv = np.float32(32767.0) / s                    # one fp32 division
        qf = np.rint(x * inv[..., None])                 # one fp32 product, ties to even
    qf = np.where((s > 0)[..., None], qf, np.float32(0.0))
    q = np.clip(qf, -32767, 32767).astype(np.int16)
    f = np.where(s > 0, s / np.float32(32767.0), np.float32(0.0)).astype(np.float32)
    return q, f


def dequantize(q, f) -> np.ndarray:
    return np.asarray(q, dtype=np.float64) * np.asarray(f, dtype=np.float64)[..., None]


def attention(q_bits, k, v, positions, scale: float):
    """Causal GQA attention of one sequence, dense.

    q_bits: bf16 [T, n_q, d] at absolute positions ``positions`` [T];
    k, v: float64 [L, n_kv, d] (row j = position j).  Returns
    (out [T, n_q, d] float64, lse [T, n_q] float64, natural log)."""
    qv = bf16_decode(q_bits)
    T, nq, d = qv.shape
    L, nkv, _ = k.shape
    group = nq // nkv
    out = np.zeros((T, nq, d))
    lse = np.zeros((T, nq))
    for t in range(T):
        p = int(positions[t])
        for h in range(nq):
            g = h // group
            z = scale * (k[:p + 1, g, :] @ qv[t, h, :])
            m = z.max()
            e = np.exp(z - m)
            out[t, h] = (e @ v[:p + 1, g, :]) / e.sum()
            lse[t, h] = m + np.log(e.sum())
    return out, lse
