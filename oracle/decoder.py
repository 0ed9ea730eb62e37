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

* ``stack_logits``: the whole pre-norm stack of these operations with
  RMSNorm, matmul and attention, teacher-forced over one sequence (below)

Inputs that are bf16 arrive as bit patterns (numpy uint16) and are widened
exactly with the oracle's own codec.  Pins: ``tests/test_oracle_decoder.py``
(group property and closed forms of the rotation, closed forms of SiLU, tie
and NaN rules of argmax) and ``tests/test_oracle_stack.py`` (the stack: zeroed
blocks and a single token in closed form, an independent torch float64
composition, and planted wiring mistakes).  Parity unpinned: nothing here is
unpinned.
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


# ---- the whole stack, teacher-forced ----------------------------------------
#
# A Llama-style pre-norm decoder evaluated for one sequence whose token ids are
# given (teacher forcing: the logits at every position, for the ids that follow
# it in the input, whatever any model would have sampled):
#
#   x_0     = embed(ids)
#   per layer:
#     h     = rmsnorm(x, attn_norm)
#     q, k  = rope(h W_q), rope(h W_k)   at positions 0..T-1;  v = h W_v
#     x     = x + attention(q, k, v) W_o          (causal, GQA)
#     h     = rmsnorm(x, mlp_norm)
#     x     = x + (silu(h W_gate) * (h W_up)) W_down
#   logits  = rmsnorm(x, final_norm) W_lm
#
# Every intermediate tensor of the stack is a bf16 tensor (the activations a
# bf16 inference stack stores between its operations), so each operation is
# evaluated exactly in float64 on bf16 inputs and its result rounded once to
# bf16 (``oracle.bf16_encode``); the logits are left in float64.  The steps
# are the oracle functions: ``oracle.rmsnorm``, ``oracle.matmul`` (bf16
# weights) or ``oracle.ec.exact`` (fp32 weights: the product the
# error-compensated matmul approximates), ``rope``, ``oracle.attention`` or,
# for an int16 cache, ``oracle.kv16`` quantisation and attention over the
# dequantised keys and values, ``swiglu`` and ``add``.
#
# The helpers below are module attributes so that a test can plant a mistake
# in one of them and see the stack's pins fail.

def _enc(x) -> np.ndarray:
    from . import bf16_encode
    return bf16_encode(x)


def _norm(x_bits, g_bits, eps) -> np.ndarray:
    from . import rmsnorm
    return _enc(rmsnorm(x_bits, g_bits, eps)[0])


def _proj(a_bits, w) -> np.ndarray:
    """a bf16 bits [T, K] times w: bf16 bits [K, N], or float32 [K, N]."""
    from . import matmul
    from . import ec
    if np.asarray(w).dtype == np.uint16:
        return matmul(a_bits, w)
    return ec.exact(bf16_decode(a_bits).astype(np.float32), w)


def _attend(q_bits, k_bits, v_bits, scale, kv16) -> np.ndarray:
    """Causal attention of one sequence at positions 0..T-1."""
    T = q_bits.shape[0]
    pos = np.arange(T)
    if kv16:
        from . import kv16 as k16
        kd = k16.dequantize(*k16.quantize(k_bits))
        vd = k16.dequantize(*k16.quantize(v_bits))
        return k16.attention(q_bits, kd, vd, pos, scale)[0]
    from . import attention
    return attention(q_bits, k_bits, v_bits, [T], [0] * T, pos, scale)[0]


def _residual(x_bits, y_bits) -> np.ndarray:
    return _enc(add(x_bits, y_bits))


def stack_logits(weights: dict, cfg, ids, kv16: bool = False) -> np.ndarray:
    """float64 logits [T, vocab] at every position of one sequence.

    weights: ``embed`` bf16 bits [vocab, hidden], ``final_norm`` bits
    [hidden], ``lm_head`` [hidden, vocab], and ``layers``, a list of dicts with
    ``attn_norm``, ``mlp_norm`` bits [hidden] and the projections ``wq``
    [hidden, n_q d], ``wk``, ``wv`` [hidden, n_kv d], ``wo`` [n_q d, hidden],
    ``w_gate``, ``w_up`` [hidden, ffn], ``w_down`` [ffn, hidden], each stored
    [in, out] as bf16 bits (uint16) or as float32 values.  cfg: any object
    with hidden, n_q, n_kv, head_dim, rope_theta and eps.  The softmax scale
    is 1/sqrt(head_dim) rounded to fp32 and eps is widened from fp32, as the
    kernels receive them.  kv16: keys and values go through the int16 cache's
    quantiser before attention."""
    ids = np.asarray(ids, dtype=np.int64)
    T = ids.size
    nq, nkv, d = cfg.n_q, cfg.n_kv, cfg.head_dim
    eps = float(np.float32(cfg.eps))
    scale = float(np.float32(1.0 / np.sqrt(d)))
    pos = np.arange(T)
    x = _enc(embed(ids, weights["embed"]))
    for lw in weights["layers"]:
        h = _norm(x, lw["attn_norm"], eps)
        q = _enc(rope(_enc(_proj(h, lw["wq"])).reshape(T, nq, d), pos, cfg.rope_theta))
        k = _enc(rope(_enc(_proj(h, lw["wk"])).reshape(T, nkv, d), pos, cfg.rope_theta))
        v = _enc(_proj(h, lw["wv"])).reshape(T, nkv, d)
        o = _enc(_attend(q, k, v, scale, kv16)).reshape(T, nq * d)
        x = _residual(x, _enc(_proj(o, lw["wo"])))
        h = _norm(x, lw["mlp_norm"], eps)
        a = _enc(swiglu(_enc(_proj(h, lw["w_gate"])), _enc(_proj(h, lw["w_up"]))))
        x = _residual(x, _enc(_proj(a, lw["w_down"])))
    return _proj(_norm(x, weights["final_norm"], eps), weights["lm_head"])
