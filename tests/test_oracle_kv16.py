"""Pins for the int16 KV-cache oracle (``oracle.kv16``).  CPU only."""
import numpy as np

import oracle
import synth
from oracle import kv16


def _bits(x):
    return synth.bf16_bits(np.asarray(x, dtype=np.float32))


def test_quantize_closed_forms():
    s = np.float32(3.0)
    x = _bits([[3.0, -3.0, 1.5, 0.0, 0.75]])
    q, f = kv16.quantize(x)
    # 1.5 * (32767/3) = 16383.5 rounds to the even 16384; 0.75 -> 8191.75 -> 8192
    assert q[0].tolist() == [32767, -32767, 16384, 0, 8192]
    assert f[0] == np.float32(s / np.float32(32767.0))
    q, f = kv16.quantize(_bits([[0.0, -0.0, 0.0, 0.0]]))
    assert q[0].tolist() == [0, 0, 0, 0] and f[0] == 0.0


def test_quantize_error_bound():
    x = synth.normal_bits((200, 8, 128), 0, 1, 0, "kv16.q")
    q, f = kv16.quantize(x)
    xd = oracle.bf16_decode(x)
    err = np.abs(kv16.dequantize(q, f) - xd)
    # half a step, plus three fp32 roundings (32767/s, the product, s/32767) of
    # relative size 2^-24 each on values up to 32767 steps: 0.5 + 32767*3*2^-24
    assert np.all(err <= (0.5 + 32767 * 3 * 2.0 ** -24) * f[..., None])
    assert np.all(np.abs(q).max(axis=-1) == 32767)


def test_dense_attention_matches_the_c_oracle():
    L, nq, nkv, d = 37, 4, 2, 16
    qb = synth.normal_bits((L, nq, d), 0, 1, 1, "kv16.aq")
    kb = synth.normal_bits((L, nkv, d), 0, 1, 1, "kv16.ak")
    vb = synth.normal_bits((L, nkv, d), 0, 1, 1, "kv16.av")
    pos = np.arange(L)
    out, lse = kv16.attention(qb, oracle.bf16_decode(kb), oracle.bf16_decode(vb), pos, 0.25)
    ref, rlse = oracle.attention(qb, kb, vb, [L], [0] * L, pos.tolist(), 0.25)
    assert np.allclose(out, ref, rtol=0, atol=1e-12) and np.allclose(lse, rlse, atol=1e-12)


def test_dense_attention_uniform_weights():
    # q = 0: every visible key weighs the same; lse = ln(p + 1)
    L, d = 9, 8
    qb = _bits(np.zeros((L, 2, d)))
    v = np.arange(L * d, dtype=np.float64).reshape(L, 1, d)
    out, lse = kv16.attention(qb, np.ones((L, 1, d)), v, np.arange(L), 1.0)
    for p in range(L):
        assert np.allclose(out[p, 0], v[:p + 1, 0].mean(axis=0), atol=1e-12)
        assert abs(lse[p, 1] - np.log(p + 1)) < 1e-12


def test_quantize_equals_exact_rint_away_from_ties():
    """The quantiser takes each integer decision in fp32 (as the kernel does).
    Against the exact code rint(32767 x / s), evaluated in float64 on the same
    bf16 inputs (where 32767 x / s is within 2^-52 of the true quotient), the
    two agree on every element except those whose exact quotient lies within
    the fp32 evaluation's error of a half-integer (two roundings of relative
    size 2^-24 on a value of at most 32767: under 0.004), and there they
    differ by one code at most.  That set is enumerated: under 1% of the
    elements here (bf16 inputs make exact ties common), of which a few
    percent actually differ."""
    x = synth.normal_bits((4000, 8, 128), 0, 1, 7, "kv16.exact")
    q, _ = kv16.quantize(x)
    xd = oracle.bf16_decode(x)
    s = np.max(np.abs(xd), axis=-1, keepdims=True)
    t = 32767.0 * xd / s
    exact = np.rint(t)
    frac = np.abs(t - np.floor(t) - 0.5)
    near = frac < 32767 * 2 * 2.0 ** -24
    diff = q.astype(np.int64) - exact.astype(np.int64)
    assert np.all(diff[~near] == 0)
    assert np.all(np.abs(diff[near]) <= 1)
    assert near.sum() < 2e-2 * x.size
    assert 0 < np.count_nonzero(diff) < 0.1 * near.sum()
    # planted: a quantiser that truncates instead of rounding breaks the pin
    trunc = np.trunc(t)
    assert np.any((trunc.astype(np.int64) - exact.astype(np.int64))[~near] != 0)
