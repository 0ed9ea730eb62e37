"""Pins for the fp64 oracle: each test ties it to something other than itself --
closed forms, hand-derived examples, exact integer arithmetic, special cases,
independent library routines (numpy / torch fp64), and the fold identity.

A plausible mistake in the oracle (eps outside the root, a mean over the wrong
count, a transposed W, a dropped scale, an off-by-one causal mask, a wrong GQA
head map, a sign error in the fold) fails at least one test here.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
EPS = float(np.float32(1e-6))  # eps passed as fp32, widened exactly


def bits(vals):
    return synth.bf16_bits(np.asarray(vals, dtype=np.float32))


def f64(b):
    return synth.bf16_to_f32(b).astype(np.float64)


# --------------------------------------------------------------------------- codec

def test_bf16_decode_all_patterns(orc):
    allb = np.arange(65536, dtype=np.uint16)
    got = orc.bf16_decode(allb)
    ref = torch.from_numpy(allb.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros survive
    assert math.copysign(1.0, got[0x8000]) == -1.0


def test_input_rounding_is_rne():
    g = np.random.default_rng(1)
    x = g.normal(0, 3, size=200000).astype(np.float32)
    # exact ties between two bf16 values, both parities
    ties = (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.bf16_bits(x), ref)


# --------------------------------------------------------------------------- RMSNorm

def test_rmsnorm_hand_examples(orc):
    ex = json.load(open(os.path.join(GOLDEN, "hand_examples.json")))
    for key in ("rmsnorm", "rmsnorm_eps"):
        e = ex[key]
        y, r = orc.rmsnorm(bits([e["x"]]), bits(e["gamma"]), e["eps"])
        np.testing.assert_allclose(r[0], e["rstd"], rtol=1e-14)
        np.testing.assert_allclose(y[0], e["y"], rtol=1e-14)


@pytest.mark.parametrize("c", [1.0, -2.5, 0.0078125, 37.0])
def test_rmsnorm_constant_row_closed_form(orc, c):
    H = 256
    gamma = synth.normal_bits((H,), 1.0, 0.1, 0, "pin.gamma")
    cb = bits([c])[0]
    x = np.full((3, H), cb, dtype=np.uint16)
    y, r = orc.rmsnorm(x, gamma, EPS)
    cv = f64([cb])[0]
    rr = 1.0 / math.sqrt(cv * cv + EPS)
    np.testing.assert_allclose(r, rr, rtol=1e-14)
    np.testing.assert_allclose(y, np.broadcast_to(cv * rr * f64(gamma), y.shape), rtol=1e-13)


def test_rmsnorm_eps_inside_root(orc):
    # c = bf16(1e-3): y = c / sqrt(c^2 + 1e-6) ~ 0.707, not ~1 (eps outside) nor 1/sqrt(H)
    H = 4096
    cb = bits([1e-3])[0]
    cv = f64([cb])[0]
    x = np.full((1, H), cb, dtype=np.uint16)
    y, _ = orc.rmsnorm(x, bits(np.ones(H)), EPS)
    expect = cv / math.sqrt(cv * cv + EPS)
    assert 0.68 < expect < 0.72
    np.testing.assert_allclose(y[0], expect, rtol=1e-13)


def test_rmsnorm_zero_row_and_spike(orc):
    H = 4096
    x = np.zeros((2, H), dtype=np.uint16)
    c = 3.0
    x[1, 17] = bits([c])[0]
    gamma = synth.normal_bits((H,), 1.0, 0.1, 0, "pin.gamma2")
    y, r = orc.rmsnorm(x, gamma, EPS)
    assert np.all(y[0] == 0.0)
    np.testing.assert_allclose(r[0], 1.0 / math.sqrt(EPS), rtol=1e-14)
    rr = 1.0 / math.sqrt(c * c / H + EPS)  # mean over all H, not over non-zeros
    np.testing.assert_allclose(r[1], rr, rtol=1e-14)
    np.testing.assert_allclose(y[1, 17], c * rr * f64(gamma)[17], rtol=1e-14)
    assert np.count_nonzero(y[1]) == 1


def test_rmsnorm_matches_torch_fp64(orc):
    for H in (256, 4096, 8192):
        x, g = synth.rmsnorm_inputs(7, H, seed=3)
        y, r = orc.rmsnorm(x, g, EPS)
        xt = torch.from_numpy(f64(x))
        ref = torch.nn.functional.rms_norm(xt, (H,), weight=torch.from_numpy(f64(g)), eps=EPS)
        np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-13)
        rref = 1.0 / torch.sqrt(xt.pow(2).mean(-1) + EPS)
        np.testing.assert_allclose(r, rref.numpy(), rtol=1e-13)


# --------------------------------------------------------------------------- matmul

def test_matmul_hand_example(orc):
    e = json.load(open(os.path.join(GOLDEN, "hand_examples.json")))["matmul"]
    c = orc.matmul(bits(e["a"]), bits(e["w"]))
    assert np.array_equal(c, np.asarray(e["c"]))


@pytest.mark.parametrize("m,n,k", [(5, 3, 7), (3, 512, 256), (2, 64, 4096)])
def test_matmul_integers_exact(orc, m, n, k):
    g = np.random.default_rng(m * 1000 + n + k)
    ai = g.integers(-4, 5, size=(m, k))
    wi = g.integers(-4, 5, size=(k, n))
    c = orc.matmul(bits(ai), bits(wi))
    assert np.array_equal(c, (ai.astype(np.int64) @ wi.astype(np.int64)).astype(np.float64))


def test_matmul_matches_numpy_and_onehot(orc):
    a, w = synth.matmul_inputs(9, 384, 256, seed=5)
    c = orc.matmul(a, w)
    ref = f64(a) @ f64(w)
    np.testing.assert_allclose(c, ref, rtol=1e-12, atol=1e-12)
    # one-hot rows of A select rows of W exactly
    oh = np.zeros((4, 256), dtype=np.uint16)
    for i, j in enumerate((0, 3, 100, 255)):
        oh[i, j] = bits([1.0])[0]
    c1 = orc.matmul(oh, w)
    assert np.array_equal(c1, f64(w)[[0, 3, 100, 255]])
    # row selection returns exactly those rows
    sel = orc.matmul(a, w, rows=[8, 0, 4])
    assert np.array_equal(sel, c[[8, 0, 4]])


# --------------------------------------------------------------------------- attention

def _flat(p: synth.AttnProblem):
    k = np.concatenate(p.k, axis=0)
    v = np.concatenate(p.v, axis=0)
    return k, v


def test_attention_hand_example(orc):
    e = json.load(open(os.path.join(GOLDEN, "hand_examples.json")))["attention"]
    q = bits([[[0.0, 0.0]], [e["q_pos1"]]])  # [2 tokens, 1 head, d=2]
    k = bits(np.asarray(e["k"])[:, None, :])
    v = bits(np.asarray(e["v"])[:, None, :])
    out, lse = orc.attention(q, k, v, [2], [0, 0], [0, 1], e["scale"])
    np.testing.assert_allclose(out[1, 0], e["out"], rtol=1e-14)
    np.testing.assert_allclose(lse[1, 0], e["lse"], rtol=1e-14)
    # position 0 sees only key 0
    assert np.array_equal(out[0, 0], f64(v)[0, 0])


def _sdpa_ref(p: synth.AttnProblem, b: int):
    """torch fp64 scaled_dot_product_attention, causal, kv heads repeated per
    group (q head h reads kv head h // group)."""
    grp = p.n_q // p.n_kv
    q = torch.from_numpy(f64(p.q[b])).permute(1, 0, 2)  # [nq, L, d]
    k = torch.from_numpy(f64(p.k[b])).permute(1, 0, 2).repeat_interleave(grp, dim=0)
    v = torch.from_numpy(f64(p.v[b])).permute(1, 0, 2).repeat_interleave(grp, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=p.scale)
    s = (q @ k.transpose(-1, -2)) * p.scale
    L = s.shape[-1]
    s = s.masked_fill(torch.triu(torch.ones(L, L, dtype=torch.bool), 1), float("-inf"))
    lse = torch.logsumexp(s, dim=-1)  # [nq, L]
    return o.permute(1, 0, 2).numpy(), lse.permute(1, 0).numpy()


def test_attention_matches_torch_sdpa_gqa(orc):
    p = synth.attn_problem([37, 300, 5], n_q=8, n_kv=2, d=64, seed=11)
    k, v = _flat(p)
    tseq, tpos, qs = [], [], []
    for b, L in enumerate(p.lens):
        tseq += [b] * L
        tpos += list(range(L))
        qs.append(p.q[b])
    out, lse = orc.attention(np.concatenate(qs), k, v, p.lens, tseq, tpos, p.scale)
    o0 = 0
    for b, L in enumerate(p.lens):
        ro, rl = _sdpa_ref(p, b)
        np.testing.assert_allclose(out[o0:o0 + L], ro, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(lse[o0:o0 + L], rl, rtol=1e-12, atol=1e-12)
        o0 += L


def test_attention_special_cases(orc):
    d, L = 64, 40
    p = synth.attn_problem([L], n_q=4, n_kv=1, d=d, seed=2)
    v = p.v[0]
    vf = f64(v)
    # Q = 0: uniform weights; lse = ln(p+1)
    q0 = np.zeros((L, 4, d), dtype=np.uint16)
    out, lse = orc.attention(q0, p.k[0], v, [L], [0] * L, list(range(L)), p.scale)
    for pos in (0, 1, 17, L - 1):
        np.testing.assert_allclose(out[pos], np.broadcast_to(vf[:pos + 1, 0].mean(0), (4, d)),
                                   rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse[pos], math.log(pos + 1), rtol=1e-13, atol=1e-15)
    # all keys equal: uniform again, lse = z + ln(p+1)
    keq = np.broadcast_to(p.k[0][:1], p.k[0].shape).copy()
    out, lse = orc.attention(p.q[0], keq, v, [L], [0] * L, list(range(L)), p.scale)
    for pos in (3, L - 1):
        z = p.scale * (f64(p.q[0][pos]) @ f64(keq[0, 0]))
        np.testing.assert_allclose(out[pos], np.broadcast_to(vf[:pos + 1, 0].mean(0), (4, d)),
                                   rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(lse[pos], z + math.log(pos + 1), rtol=1e-12)
    # position 0 sees only key 0: out == V[0] bitwise, lse = z_0
    out, lse = orc.attention(p.q[0][:1], p.k[0], v, [L], [0], [0], p.scale)
    assert np.array_equal(out[0], np.broadcast_to(vf[0, 0], (4, d)))
    np.testing.assert_allclose(lse[0], p.scale * (f64(p.q[0][0]) @ f64(p.k[0][0, 0])), rtol=1e-14)


def test_attention_dominant_key(orc):
    d, L, j = 64, 50, 23
    g = np.random.default_rng(4)
    kf = np.zeros((L, 1, d), dtype=np.float32)
    kf[np.arange(L), 0, np.arange(L) % d] = 1.0  # orthonormal-ish keys
    qf = np.zeros((1, 1, d), dtype=np.float32)
    qf[0, 0, j % d] = 64.0
    v = bits(g.normal(size=(L, 1, d)))
    out, _ = orc.attention(bits(qf), bits(kf), v, [L], [0], [L - 1], 1.0)
    # weight of key j is ~1 - L e^-64; the others ~e^-64 each
    np.testing.assert_allclose(out[0, 0], f64(v)[j, 0], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("split", [1, 16, 256])
def test_attention_fold_identity(orc, split):
    """Split-and-fold over fixed blocks at absolute multiples equals the direct
    definition (pins the combine algebra: max update, both rescale factors)."""
    lens = [700, 257, 1]
    p = synth.attn_problem(lens, n_q=4, n_kv=2, d=32, seed=8)
    k, v = _flat(p)
    tseq = [0, 0, 0, 0, 0, 0, 1, 1, 1, 2]
    tpos = [0, 255, 256, 257, 511, 699, 0, 255, 256, 0]
    q = np.stack([p.q[b][t] for b, t in zip(tseq, tpos)])
    o1, l1 = orc.attention(q, k, v, lens, tseq, tpos, p.scale)
    o2, l2 = orc.attention(q, k, v, lens, tseq, tpos, p.scale, split=split)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=1e-13, atol=1e-13)


def test_attention_query_subset_independent(orc):
    """A query's result does not depend on which other queries share the call."""
    lens = [90, 60]
    p = synth.attn_problem(lens, n_q=4, n_kv=2, d=32, seed=9)
    k, v = _flat(p)
    q = np.stack([p.q[0][89], p.q[1][10], p.q[0][3]])
    oa, la = orc.attention(q, k, v, lens, [0, 1, 0], [89, 10, 3], p.scale)
    ob, lb = orc.attention(q[1:2], k, v, lens, [1], [10], p.scale)
    assert np.array_equal(oa[1], ob[0]) and np.array_equal(la[1], lb[0])
