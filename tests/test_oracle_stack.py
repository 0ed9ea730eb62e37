"""Pins for the oracle's whole-stack forward (``oracle.decoder.stack_logits``)
and for the codec that rounds its intermediate tensors to bf16
(``oracle.bf16_encode``).  CPU only.

* the encoder: all 65,536 patterns round-trip; fp32 inputs round as torch's
  own fp32 -> bf16 conversion does; hand cases for ties, a value just past a
  tie that fp32 cannot hold (a double rounding would miss it), gradual
  underflow and overflow;
* the stack, in closed form: with every attention and MLP output projection
  zero the residual stream is the embedding, so the logits are
  rmsnorm(embedding) times the lm_head; a single token attends only to itself
  (weight exactly 1), so one layer adds bf16(bf16(v) W_o) with v the token's
  value row of its kv head;
* the stack against an independent float64 composition in torch (F.rms_norm,
  scaled_dot_product_attention with causal masking and grouped kv heads,
  F.silu, the rotation as a complex product) rounded at the same points;
* planted mistakes in the oracle (rotation dropped, gate and up swapped, a
  residual dropped, attention without its causal mask, kv heads assigned
  h mod n_kv, the final norm dropped, the int16 quantiser skipped) each fail
  that comparison."""
from types import SimpleNamespace

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
import oracle
from oracle import decoder as od

CFG = SimpleNamespace(hidden=64, layers=2, n_q=4, n_kv=2, head_dim=16, ffn=96, vocab=80,
                      rope_theta=10000.0, eps=1e-5)


def _weights(fp32=False, seed=0):
    c = CFG
    return synth.llama_weights_host(c.hidden, c.layers, c.n_q, c.n_kv, c.head_dim, c.ffn,
                                    c.vocab, seed=seed, fp32=fp32)


def _val(w):
    w = np.asarray(w)
    return oracle.bf16_decode(w) if w.dtype == np.uint16 else w.astype(np.float64)


def _rel(g, o):
    g, o = np.asarray(g, np.float64), np.asarray(o, np.float64)
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True))
    return float(np.max(np.abs(g - o) / np.maximum(np.abs(o), rms)))


# ---- the bf16 encoder ----------------------------------------------------------

def test_encode_round_trips_every_pattern():
    b = np.arange(65536, dtype=np.uint16)
    v = oracle.bf16_decode(b)
    ok = ~np.isnan(v)
    assert np.array_equal(oracle.bf16_encode(v[ok]), b[ok])
    assert np.all(np.isnan(oracle.bf16_decode(oracle.bf16_encode(v[~ok]))))


def test_encode_matches_torch_on_fp32_values():
    rng = synth.stream(0, "enc.torch")
    x = (rng.standard_normal(200000) * 10.0 ** rng.integers(-44, 38, 200000)).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_encode(x.astype(np.float64)), want)


def test_encode_rounds_once():
    e = lambda v: int(oracle.bf16_encode([v])[0])
    assert e(1.0 + 2.0 ** -8) == 0x3F80               # tie -> even (1.0)
    assert e(1.0 + 3 * 2.0 ** -8) == 0x3F82           # tie -> even (1 + 2^-6)
    assert e(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81  # just past the tie: up (fp32 would tie)
    assert e(-(1.0 + 2.0 ** -8 + 2.0 ** -40)) == 0xBF81
    assert e(2.0 ** -133) == 0x0001 and e(2.0 ** -134) == 0x0000 and e(3 * 2.0 ** -134) == 0x0002
    assert e(3.4e38) == 0x7F80 and e(-3.4e38) == 0xFF80 and e(3.38e38) == 0x7F7E
    assert e(-0.0) == 0x8000 and e(float("inf")) == 0x7F80


# ---- the stack in closed form --------------------------------------------------

def _rms(x, g, eps):
    return oracle.bf16_encode(x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g)


def test_zeroed_blocks_pass_the_embedding_through():
    w = _weights()
    for lw in w["layers"]:
        lw["wo"] = np.zeros_like(lw["wo"])
        lw["w_down"] = np.zeros_like(lw["w_down"])
    ids = synth.stream(1, "st.ids").integers(0, CFG.vocab, size=9)
    got = od.stack_logits(w, CFG, ids)
    x = oracle.bf16_decode(w["embed"])[ids]
    eps = float(np.float32(CFG.eps))
    y = oracle.bf16_decode(_rms(x, oracle.bf16_decode(w["final_norm"]), eps))
    want = y @ _val(w["lm_head"])
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("fp32", [False, True])
def test_single_token_attends_to_itself(fp32):
    """One token at position 0, one layer, the MLP's output projection zero:
    x1 = bf16(x + bf16(o W_o)), o's head h = bf16(h W_v) of kv head h // 2."""
    w = _weights(fp32=fp32)
    w["layers"] = w["layers"][:1]
    w["layers"][0]["w_down"] = np.zeros_like(w["layers"][0]["w_down"])
    cfg = SimpleNamespace(**dict(vars(CFG), layers=1))
    tok = 37
    got = od.stack_logits(w, cfg, [tok])
    lw = w["layers"][0]
    eps = float(np.float32(CFG.eps))
    enc, dec = oracle.bf16_encode, oracle.bf16_decode
    x = dec(w["embed"])[tok][None, :]
    h = dec(_rms(x, dec(lw["attn_norm"]), eps))
    v = dec(enc(h @ _val(lw["wv"]))).reshape(CFG.n_kv, CFG.head_dim)
    o = np.stack([v[hq // (CFG.n_q // CFG.n_kv)] for hq in range(CFG.n_q)]).reshape(1, -1)
    x1 = dec(enc(x + dec(enc(o @ _val(lw["wo"])))))
    want = dec(_rms(x1, dec(w["final_norm"]), eps)) @ _val(w["lm_head"])
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


# ---- the stack against an independent torch composition ---------------------------

def _torch_stack(w, cfg, ids, kv16=False):
    """float64 torch: F.rms_norm, causal SDPA with grouped kv heads, F.silu,
    rotation as a complex product; intermediates rounded to bf16 through
    fp32 (a double rounding: it can differ from a single one by one bf16 step
    on a value within 2^-24 of a tie, which these tolerances absorb)."""
    t = lambda a: torch.from_numpy(_val(a))
    rb = lambda x: x.to(torch.float32).to(torch.bfloat16).to(torch.float64)
    T, H, nq, nkv, d = len(ids), cfg.hidden, cfg.n_q, cfg.n_kv, cfg.head_dim
    eps = float(np.float32(cfg.eps))
    scale = float(np.float32(1.0 / np.sqrt(d)))
    ang = torch.arange(T, dtype=torch.float64)[:, None] * \
        cfg.rope_theta ** (-torch.arange(0, d, 2, dtype=torch.float64) / d)[None, :]
    rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]          # [T, 1, d/2]

    def rope(x):                                                      # pairs (i, i + d/2)
        z = torch.complex(x[..., :d // 2], x[..., d // 2:]) * rot
        return torch.cat([z.real, z.imag], dim=-1)

    def quant(x):                                                     # per (token, head) int16
        s = x.abs().amax(-1, keepdim=True).to(torch.float32)
        big = torch.full_like(s, 32767.0)      # (a scalar / tensor goes through a reciprocal)
        q = torch.round(x.to(torch.float32) * (big / s))
        return q.to(torch.float64) * (s / big).to(torch.float64)

    x = t(w["embed"])[torch.as_tensor(ids)]
    for lw in w["layers"]:
        h = rb(F.rms_norm(x, (H,), t(lw["attn_norm"]), eps))
        q = rb(rope(rb(h @ t(lw["wq"])).view(T, nq, d)))
        k = rb(rope(rb(h @ t(lw["wk"])).view(T, nkv, d)))
        v = rb(h @ t(lw["wv"])).view(T, nkv, d)
        if kv16:
            k, v = quant(k), quant(v)
        o = F.scaled_dot_product_attention(q.transpose(0, 1)[None], k.transpose(0, 1)[None],
                                           v.transpose(0, 1)[None], is_causal=True, scale=scale,
                                           enable_gqa=True)
        o = rb(o[0].transpose(0, 1).reshape(T, nq * d))
        x = rb(x + rb(o @ t(lw["wo"])))
        h = rb(F.rms_norm(x, (H,), t(lw["mlp_norm"]), eps))
        a = rb(F.silu(rb(h @ t(lw["w_gate"]))) * rb(h @ t(lw["w_up"])))
        x = rb(x + rb(a @ t(lw["w_down"])))
    return (rb(F.rms_norm(x, (H,), t(w["final_norm"]), eps)) @ t(w["lm_head"])).numpy()


IDS = synth.stream(2, "st.ids2").integers(0, CFG.vocab, size=24)
TOL = 1e-3


@pytest.mark.parametrize("fp32,kv16", [(False, False), (True, False), (False, True)])
def test_stack_matches_torch_composition(fp32, kv16):
    w = _weights(fp32=fp32, seed=3)
    got = od.stack_logits(w, CFG, IDS, kv16=kv16)
    want = _torch_stack(w, CFG, IDS, kv16=kv16)
    assert got.shape == (len(IDS), CFG.vocab)
    assert _rel(got, want) < TOL


def _plant(monkeypatch, which):
    """Put one plausible mistake into the oracle."""
    if which == "rope dropped":
        monkeypatch.setattr(od, "rope", lambda x, pos, theta: od._f64(x))
    elif which == "gate and up swapped":
        sw = od.swiglu
        monkeypatch.setattr(od, "swiglu", lambda g, u: sw(u, g))
    elif which == "residual dropped":
        monkeypatch.setattr(od, "_residual", lambda x, y: y)
    elif which == "no causal mask":
        att = oracle.attention
        monkeypatch.setattr(oracle, "attention", lambda q, k, v, lens, ts, tp, sc: att(
            q, k, v, lens, ts, [lens[0] - 1] * len(tp), sc))
    elif which == "kv head h mod n_kv":
        att = oracle.attention

        def mod_map(q, k, v, lens, ts, tp, sc):
            # query head h reads kv head h % n_kv instead of h // group
            nq, nkv = q.shape[1], k.shape[1]
            perm = [h % nkv * (nq // nkv) + h // nkv for h in range(nq)]
            out, lse = att(q[:, perm], k, v, lens, ts, tp, sc)
            inv = np.argsort(perm)
            return out[:, inv], lse[:, inv]
        monkeypatch.setattr(oracle, "attention", mod_map)
    elif which == "final norm dropped":
        nm = od._norm
        monkeypatch.setattr(od, "_norm", lambda x, g, eps: x if g is FINAL[0] else nm(x, g, eps))


FINAL = [None]


@pytest.mark.parametrize("which", ["rope dropped", "gate and up swapped", "residual dropped",
                                   "no causal mask", "kv head h mod n_kv", "final norm dropped"])
def test_planted_mistakes_fail_the_comparison(monkeypatch, which):
    w = _weights(seed=3)
    FINAL[0] = w["final_norm"]
    want = _torch_stack(w, CFG, IDS)
    _plant(monkeypatch, which)
    got = od.stack_logits(w, CFG, IDS)
    assert _rel(got, want) > 50 * TOL, which


def test_skipping_the_int16_quantiser_fails_the_kv16_comparison():
    """The codes move each key and value by at most half a code step (2^-16 of
    the row's largest magnitude), but through the bf16 roundings after them
    that moves the logits well past the bar."""
    w = _weights(seed=3)
    want = _torch_stack(w, CFG, IDS, kv16=True)
    assert _rel(od.stack_logits(w, CFG, IDS, kv16=True), want) < TOL
    assert _rel(od.stack_logits(w, CFG, IDS, kv16=False), want) > 10 * TOL
