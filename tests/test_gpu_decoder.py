"""The decoder-stack kernels (embedding gather, rotary embedding, SwiGLU,
residual add, argmax) against the fp64 oracle, and the end-to-end property:
a sequence's greedy tokens and logits are bitwise the same alone, among other
sequences, and under chunked prefill."""
import numpy as np
import pytest
import torch

import synth
from helpers import TOL_BF16, dev, rel_err
import invariant_bi_matmul_amd as bi
from invariant_bi_matmul_amd.model import Decoder, LlamaConfig
from oracle import decoder as od

pytestmark = pytest.mark.gpu


def _t(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev()).view(torch.bfloat16)


def _np(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def test_embed_is_an_exact_gather():
    table = synth.normal_bits((1000, 256), 0, 1, 0, "dec.embed")
    ids = np.array([0, 999, 17, 17, -3, 1000, 5000, 512], dtype=np.int32)
    got = bi.embed(torch.from_numpy(ids).to(dev()), _t(table))
    assert np.array_equal(synth.bf16_to_f32(_np(got)).astype(np.float64), od.embed(ids, table))


@pytest.mark.parametrize("theta", [10000.0, 500000.0])
def test_rope_parity(theta):
    T = 37
    q = synth.normal_bits((T, 4, 64), 0, 1, 1, "dec.rq")
    k = synth.normal_bits((T, 2, 64), 0, 1, 1, "dec.rk")
    pos = synth.stream(1, "dec.rpos").integers(0, 32768, size=T).astype(np.int32)
    pos[0] = 0
    qt, kt = _t(q), _t(k)
    bi.rope(qt, kt, torch.from_numpy(pos).to(dev()), theta)
    assert rel_err(synth.bf16_to_f32(_np(qt)), od.rope(q, pos, theta)) < TOL_BF16
    assert rel_err(synth.bf16_to_f32(_np(kt)), od.rope(k, pos, theta)) < TOL_BF16
    # position 0 is the identity, bit for bit
    assert np.array_equal(_np(qt)[0], q[0]) and np.array_equal(_np(kt)[0], k[0])


def test_rope_row_does_not_depend_on_the_call():
    q = synth.normal_bits((64, 4, 128), 0, 1, 2, "dec.rq2")
    k = synth.normal_bits((64, 2, 128), 0, 1, 2, "dec.rk2")
    pos = np.arange(1000, 1064, dtype=np.int32)
    qa, ka = _t(q), _t(k)
    bi.rope(qa, ka, torch.from_numpy(pos).to(dev()), 500000.0)
    qb, kb = _t(q[40:41]), _t(k[40:41])
    bi.rope(qb, kb, torch.from_numpy(pos[40:41]).to(dev()), 500000.0)
    assert torch.equal(qa[40:41].view(torch.int16), qb.view(torch.int16))
    assert torch.equal(ka[40:41].view(torch.int16), kb.view(torch.int16))


def test_swiglu_and_add_parity():
    n = 8 * 4099
    g = synth.normal_bits((n,), 0, 3, 3, "dec.g")
    u = synth.normal_bits((n,), 0, 1, 3, "dec.u")
    got = bi.swiglu(_t(g), _t(u))
    assert rel_err(synth.bf16_to_f32(_np(got)), od.swiglu(g, u)) < TOL_BF16
    got = bi.add(_t(g), _t(u))
    assert rel_err(synth.bf16_to_f32(_np(got)), od.add(g, u)) < TOL_BF16
    a = _t(g)
    bi.add(a, _t(u), out=a)  # in place, as the residual stream uses it
    assert torch.equal(a.view(torch.int16), got.view(torch.int16))


def test_argmax_matches_the_oracle_exactly():
    rng = synth.stream(4, "dec.am")
    x = rng.standard_normal((40, 128256)).astype(np.float32)
    x[1, [5, 77, 90000]] = 9.0                 # tie: lowest index wins
    x[2, :] = np.nan
    x[2, 12345] = -1.0                         # NaNs never chosen
    x[3, :] = np.nan                           # nothing to choose: 0
    x[4, :] = -np.inf
    x[5, [3, 100000]] = np.inf
    got = bi.argmax(torch.from_numpy(x).to(dev())).cpu().numpy()
    ref = od.argmax(x)
    assert ref[1] == 5 and ref[2] == 12345 and ref[3] == 0 and ref[4] == 0 and ref[5] == 3
    assert np.array_equal(got, ref)


# ---- the stack -----------------------------------------------------------------

TOY = LlamaConfig(hidden=256, layers=2, n_q=4, n_kv=2, head_dim=64, ffn=512, vocab=1024,
                  rope_theta=10000.0)


def _weights(cfg, seed=0):
    return synth.llama_weights(cfg.hidden, cfg.layers, cfg.n_q, cfg.n_kv, cfg.head_dim, cfg.ffn,
                               cfg.vocab, seed=seed)


def _same(a, b):
    return all(torch.equal(x.view(torch.int32), y.view(torch.int32)) for x, y in zip(a, b)) \
        and len(a) == len(b)


def test_toy_stack_alone_batched_and_chunked_are_bitwise_equal():
    w = _weights(TOY)
    probe = synth.token_ids(250, TOY.vocab, 0, "dec.probe")      # decode crosses position 256
    others = {7: synth.token_ids(17, TOY.vocab, 0, "dec.c1"),
              3: synth.token_ids(300, TOY.vocab, 0, "dec.c2"),
              9: synth.token_ids(64, TOY.vocab, 0, "dec.c3")}
    steps = 12
    alone = Decoder(TOY, w, max_tokens=4096).generate({0: probe}, steps, keep_logits=[0])
    batch = {7: others[7], 0: probe, 3: others[3], 9: others[9]}
    together = Decoder(TOY, w, max_tokens=4096).generate(batch, steps, keep_logits=[0])
    chunked = Decoder(TOY, w, max_tokens=4096).generate({0: probe}, steps, chunk=32,
                                                        keep_logits=[0])
    assert len(alone[0][0]) == steps
    assert alone[0][0] == together[0][0] == chunked[0][0]
    assert _same(alone[1][0], together[1][0]) and _same(alone[1][0], chunked[1][0])


@pytest.mark.parametrize("comparator", [False, True])
def test_graph_decode_equals_eager(comparator):
    """Decode steps replayed from a captured graph give the eager steps' tokens
    and logits bit for bit (the comparator too: its splits follow the batch,
    which a graph keeps fixed)."""
    w = _weights(TOY, seed=2)
    batch = {5: synth.token_ids(40, TOY.vocab, 2, "g.a"),
             1: synth.token_ids(270, TOY.vocab, 2, "g.b"),
             8: synth.token_ids(3, TOY.vocab, 2, "g.c")}
    runs = [Decoder(TOY, w, max_tokens=4096, comparator=comparator).generate(
        batch, 20, keep_logits=[5, 1, 8], graph=g) for g in (False, True)]
    for sid in batch:
        assert runs[0][0][sid] == runs[1][0][sid], sid
        assert _same(runs[0][1][sid], runs[1][1][sid]), sid


def test_fused_projections_equal_separate_ones():
    """q|k|v and gate|up as one matmul each (then bi_qkv_rope and
    bi_swiglu_pair) give the separate projections' tokens and logits bit for
    bit, in prefill and decode."""
    w = _weights(TOY, seed=3)
    batch = {2: synth.token_ids(70, TOY.vocab, 3, "f.a"),
             4: synth.token_ids(300, TOY.vocab, 3, "f.b")}
    runs = [Decoder(TOY, w, max_tokens=4096, fuse=f).generate(batch, 6, chunk=64,
                                                              keep_logits=[2, 4])
            for f in (False, True)]
    for sid in batch:
        assert runs[0][0][sid] == runs[1][0][sid], sid
        assert _same(runs[0][1][sid], runs[1][1][sid]), sid


def test_qkv_rope_and_swiglu_pair_match_the_separate_kernels():
    T, nq, nkv, d = 37, 8, 2, 64
    qkv = synth.device_normal_bf16((T, (nq + 2 * nkv) * d), 0.0, 2.0, 4, "f.qkv", dev())
    pos = torch.arange(1000, 1000 + T, dtype=torch.int32, device=dev())
    q, k, v = bi.qkv_rope(qkv, pos, nq, nkv, 500000.0)
    rows = qkv.view(T, nq + 2 * nkv, d)
    q2, k2 = rows[:, :nq].contiguous(), rows[:, nq:nq + nkv].contiguous()
    bi.rope(q2, k2, pos, 500000.0)
    assert torch.equal(q.view(torch.int16), q2.view(torch.int16))
    assert torch.equal(k.view(torch.int16), k2.view(torch.int16))
    assert torch.equal(v.view(torch.int16), rows[:, nq + nkv:].contiguous().view(torch.int16))
    gu = synth.device_normal_bf16((T, 2 * 512), 0.0, 3.0, 4, "f.gu", dev())
    got = bi.swiglu_pair(gu)
    want = bi.swiglu(gu[:, :512].contiguous(), gu[:, 512:].contiguous())
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))


def test_stack_logits_follow_the_argmax_rule():
    w = _weights(TOY, seed=1)
    toks, logits = Decoder(TOY, w, max_tokens=1024).generate(
        {0: synth.token_ids(40, TOY.vocab, 1, "dec.p")}, 4, keep_logits=[0])
    for t, lg in zip(toks[0], logits[0]):
        assert t == int(od.argmax(lg.cpu().numpy()[None, :])[0])


def test_llama8b_shaped_stack_alone_vs_63_companions():
    """Llama-3-8B shape (32 layers, hidden 4096, GQA 32/8, SwiGLU 14336, vocab
    128256), random-init weights: a 256-token random prompt decoded greedily
    for 128 tokens alone and among 63 other random prompts (lengths 64..512)
    gives the same tokens and bitwise the same logits at every step.  With the
    non-invariant comparator kernels the logits differ (negative control)."""
    cfg = LlamaConfig()
    w = _weights(cfg)
    probe = synth.token_ids(256, cfg.vocab, 0, "e2e.probe")
    lens = synth.stream(0, "e2e.lens").integers(64, 513, size=63).tolist()
    batch = {i + 1: synth.token_ids(L, cfg.vocab, 0, "e2e.c%d" % i) for i, L in enumerate(lens)}
    batch[0] = probe  # in the middle of the batch order
    for i in range(40, 64):
        batch[i] = batch.pop(i)
    steps, cap = 128, 64 * (512 + 128) + 64
    dec = Decoder(cfg, w, max_tokens=cap)
    a_tok, a_log = dec.generate({0: probe}, steps, keep_logits=[0])
    b_tok, b_log = dec.generate(batch, steps, keep_logits=[0])
    assert len(a_tok[0]) == steps and a_tok[0] == b_tok[0]
    assert _same(a_log[0], b_log[0])
    del dec
    comp = Decoder(cfg, w, max_tokens=cap, comparator=True)
    c_tok, c_log = comp.generate({0: probe}, 2, keep_logits=[0])
    d_tok, d_log = comp.generate(batch, 2, keep_logits=[0])
    assert not _same(c_log[0], d_log[0])
