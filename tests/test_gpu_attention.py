"""Paged attention on the GPU: parity with the fp64 oracle and bitwise
invariance across chunkings, prefill vs decode, batch companions, batch
position and physical page placement."""
import numpy as np
import pytest

import synth
from helpers import (TOL_BF16, TOL_F32, PagedRun, f64, lse_err, oracle_attention, rel_err)

pytestmark = pytest.mark.gpu


def _parity(orc, prob, run, picks):
    out, lse = oracle_attention(orc, prob, picks)
    got = np.stack([run.out[b][p] for b, p in picks])
    glse = np.stack([run.lse[b][p] for b, p in picks])
    assert rel_err(f64(got), out) < TOL_BF16
    assert lse_err(glse, lse) < TOL_F32


# ---- toy decoder block: 4 heads, d=64, causal, seq 128 ------------------------

@pytest.mark.parametrize("B", [1, 3, 8])
def test_toy_whole_vs_chunks_of_32(orc, B):
    prob = synth.attn_problem([128] * B, n_q=4, n_kv=4, d=64, seed=0)
    whole = PagedRun(prob, page_seed=1)
    whole.prefill([(b, 128) for b in range(B)])
    chunked = PagedRun(prob, page_seed=2)
    chunked.run_chunked(32)
    for b in range(B):
        assert np.array_equal(whole.out[b], chunked.out[b])
        assert np.array_equal(whole.lse[b].view(np.uint32), chunked.lse[b].view(np.uint32))
    _parity(orc, prob, whole, [(b, p) for b in range(B) for p in range(128)])


def test_toy_row0_across_batch_sizes():
    ref = None
    for B in (1, 3, 8):
        prob = synth.attn_problem([128] * B, n_q=4, n_kv=4, d=64, seed=0)
        run = PagedRun(prob, page_seed=B)
        run.run_chunked(32 if B == 3 else 128)
        if ref is None:
            ref = run.out[0].copy()
        assert np.array_equal(run.out[0], ref)


# ---- GQA 32/8, d=128 ------------------------------------------------------------

def _gqa(lens, seed=0, tags=None):
    return synth.attn_problem(lens, n_q=32, n_kv=8, d=128, seed=seed, tags=tags)


BOUNDARY = (0, 1, 255, 256, 257, 511)


def test_gqa_512_chunkings_and_decode_equal_one_shot(orc):
    lens, _ = synth.ragged_lengths(4, 512, seed=0)
    prob = _gqa(lens)
    one = PagedRun(prob, page_seed=10)
    one.prefill([(b, L) for b, L in enumerate(lens)])
    picks = [(b, p) for b, L in enumerate(lens) for p in BOUNDARY + (L - 1,) if p < L]
    _parity(orc, prob, one, picks)
    for chunk in (512, 128, 100, 33, 1):
        run = PagedRun(prob, page_seed=11 + chunk)
        run.run_chunked(chunk)
        for b in range(len(lens)):
            assert np.array_equal(run.out[b], one.out[b]), (chunk, b)
            assert np.array_equal(run.lse[b].view(np.uint32), one.lse[b].view(np.uint32))
    # prefill most of each sequence, then decode the rest one token per call
    dec = PagedRun(prob, page_seed=99)
    dec.prefill([(b, L - 40) for b, L in enumerate(lens)])
    for _ in range(40):
        dec.decode(list(range(len(lens))))
    for b in range(len(lens)):
        assert np.array_equal(dec.out[b], one.out[b]), b
        assert np.array_equal(dec.lse[b].view(np.uint32), one.lse[b].view(np.uint32))


def test_gqa_4096_chunked_prefill_then_decode(orc):
    lens = [4096, 3001]
    prob = _gqa(lens, seed=1)
    one = PagedRun(prob, page_seed=3)
    one.prefill([(b, L) for b, L in enumerate(lens)])
    picks = [(0, p) for p in (0, 255, 256, 1023, 2048, 4095)] + [(1, 3000), (1, 2999)]
    _parity(orc, prob, one, picks)
    run = PagedRun(prob, page_seed=4)
    # 512-token chunks for all but the last 16 tokens, which are decoded
    while True:
        items = [(b, min(512, L - 16 - run.cur[b])) for b, L in enumerate(lens)
                 if run.cur[b] < L - 16]
        if not items:
            break
        run.prefill(items)
    for _ in range(16):
        run.decode([0, 1])
    for b in range(2):
        assert np.array_equal(run.out[b], one.out[b])


@pytest.mark.parametrize("nq,nkv,d,L,B", [(8, 2, 64, 1024, 16), (4, 4, 64, 2048, 16),
                                          (32, 8, 128, 1024, 8)])
def test_wide_prefill_equals_narrow_chunks(orc, nq, nkv, d, L, B):
    """A one-shot prefill with enough queries runs two query blocks per wave;
    small chunks run one.  Both give the same bits, and match the oracle."""
    lens, _ = synth.ragged_lengths(B, L, seed=3)
    prob = synth.attn_problem(lens, n_q=nq, n_kv=nkv, d=d, seed=4)
    wide = PagedRun(prob, page_seed=1)
    wide.prefill([(b, n) for b, n in enumerate(lens)])
    narrow = PagedRun(prob, page_seed=2)
    narrow.run_chunked(64)
    for b in range(B):
        assert np.array_equal(wide.out[b], narrow.out[b]), b
        assert np.array_equal(wide.lse[b].view(np.uint32), narrow.lse[b].view(np.uint32)), b
    picks = [(b, p) for b in (0, B - 1) for p in (0, 255, 256, lens[b] - 1)]
    _parity(orc, prob, wide, picks)


def test_decode_batch_companions_and_position():
    """A probe sequence's decode rows are the same alone and among 15
    companions at any batch index, with different page placements."""
    L = 1000
    comp_lens, _ = synth.ragged_lengths(15, 1024, seed=5)
    results = []
    for idx, page_seed in ((None, 0), (0, 1), (7, 2), (15, 3)):
        if idx is None:
            lens, tags = [L], ["probe"]
        else:
            lens = comp_lens[:idx] + [L] + comp_lens[idx:]
            tags = ["c%d" % i for i in range(idx)] + ["probe"] + ["c%d" % i for i in range(idx, 15)]
        prob = _gqa(lens, seed=7, tags=tags)
        run = PagedRun(prob, page_seed=page_seed)
        run.prefill([(b, n - 3) for b, n in enumerate(lens)])
        for _ in range(3):
            run.decode(list(range(len(lens))))
        pb = 0 if idx is None else idx
        results.append(run.out[pb][L - 3:].copy())
    for r in results[1:]:
        assert np.array_equal(r, results[0])


@pytest.mark.parametrize("nq,nkv,d", [(32, 8, 128), (8, 2, 64), (4, 4, 64)])
def test_decode_append_writes_exactly_the_new_rows(nq, nkv, d):
    """The decode call appends its token inside the split pass.  After one
    decode step every pool row is what it was, except each sequence's new
    position, which holds that token's key and value rows bitwise: new
    positions 0, 255 (the last key of a full split), 256 (a split's first
    key), mid-split, 511 and 4095.  Unused pages stay NaN-poisoned."""
    from helpers import bits_of
    lens = [1, 256, 257, 300, 512, 4096]
    prob = synth.attn_problem(lens, n_q=nq, n_kv=nkv, d=d, seed=11)
    run = PagedRun(prob, page_seed=4)
    run.prefill([(b, L - 1) for b, L in enumerate(lens) if L > 1])
    k_before, v_before = bits_of(run.kc), bits_of(run.vc)
    run.decode(list(range(len(lens))))
    want_k, want_v = k_before.copy(), v_before.copy()
    for b, L in enumerate(lens):
        pos = L - 1
        page = run.bt_host[b, pos // 16]
        want_k[page, :, pos % 16, :] = prob.k[b][pos]
        want_v[page, :, pos % 16, :] = prob.v[b][pos]
    assert np.array_equal(bits_of(run.kc), want_k)
    assert np.array_equal(bits_of(run.vc), want_v)
    # and the rows the step attended over include the new one: its output
    # equals a one-shot prefill of the whole sequence
    one = PagedRun(prob, page_seed=5)
    one.prefill([(b, L) for b, L in enumerate(lens)])
    for b, L in enumerate(lens):
        assert np.array_equal(run.out[b][L - 1], one.out[b][L - 1]), b


def test_long_context_32768(orc):
    L = 32768
    prob = _gqa([L], seed=9)
    one = PagedRun(prob, page_seed=5)
    one.prefill([(0, L)])
    picks = [(0, p) for p in (0, 256, 4096, 20000, 32767)]
    _parity(orc, prob, one, picks)
    dec = PagedRun(prob, page_seed=6)
    dec.run_chunked(8192)
    assert np.array_equal(dec.out[0], one.out[0])
    tail = PagedRun(prob, page_seed=7)
    tail.prefill([(0, L - 2)])
    tail.decode([0])
    tail.decode([0])
    assert np.array_equal(tail.out[0][L - 2:], one.out[0][L - 2:])


def _chunks_then_decode(run, lens, chunk, tail):
    """Prefill every sequence to len - tail in calls of `chunk` tokens per
    sequence (all sequences with tokens left in each call), then `tail`
    decode steps of the whole batch."""
    B = len(lens)
    while True:
        items = [(b, min(chunk, lens[b] - tail - run.cur[b])) for b in range(B)
                 if run.cur[b] < lens[b] - tail]
        if not items:
            break
        run.prefill(items)
    for _ in range(tail):
        run.decode(list(range(B)))


def test_long_context_32768_in_512_token_chunks(orc):
    """The attention workload's chunking at L = 32768: 512-token chunks, then
    decode steps, equal one-shot prefill bit for bit (GQA 32/8, d=128)."""
    L = 32768
    prob = _gqa([L], seed=9)
    one = PagedRun(prob, page_seed=5)
    one.prefill([(0, L)])
    ch = PagedRun(prob, page_seed=11)
    _chunks_then_decode(ch, [L], 512, 4)
    assert np.array_equal(ch.out[0], one.out[0])
    assert np.array_equal(ch.lse[0].view(np.uint32), one.lse[0].view(np.uint32))
    _parity(orc, prob, ch, [(0, p) for p in (511, 512, 16383, 32764, 32767)])


def test_ragged_batch_up_to_32768_in_512_token_chunks(orc):
    """A ragged batch whose longest sequence holds 32768 positions (the
    others 9000 and 20001): 512-token chunks of the whole batch per call,
    then decode steps, equal each sequence's one-shot prefill bit for bit.
    8 q heads over 2 kv heads (group 4, d=128) keep the host inputs small."""
    lens = [9000, 32768, 20001]
    prob = synth.attn_problem(lens, n_q=8, n_kv=2, d=128, seed=13,
                              tags=["rg%d" % i for i in range(3)])
    one = PagedRun(prob, page_seed=3)
    one.prefill([(b, L) for b, L in enumerate(lens)])
    ch = PagedRun(prob, page_seed=4)
    _chunks_then_decode(ch, lens, 512, 3)
    for b in range(3):
        assert np.array_equal(ch.out[b], one.out[b]), b
        assert np.array_equal(ch.lse[b].view(np.uint32), one.lse[b].view(np.uint32)), b
    _parity(orc, prob, ch, [(0, 8999), (1, 32767), (1, 12345), (2, 20000), (2, 256)])


def test_pins_position0_and_uniform(orc):
    d, nq, nkv = 128, 32, 8
    L = 300
    q, k, v = synth.attn_seq(L, nq, nkv, d, seed=3, tag="pin")
    prob = synth.AttnProblem([L], nq, nkv, d, [np.zeros_like(q)], [k], [v])
    run = PagedRun(prob, page_seed=8)
    run.prefill([(0, L)])
    grp = nq // nkv
    # position 0: weight exactly 1 on key 0 -> out == V[0] bitwise
    for h in range(nq):
        assert np.array_equal(run.out[0][0, h], v[0, h // grp])
    # Q = 0: uniform weights, lse = ln(p + 1)
    for p in (1, 255, 256, 299):
        mean = f64(v[:p + 1]).mean(axis=0)  # [nkv, d]
        expect = np.repeat(mean, grp, axis=0)
        assert rel_err(f64(run.out[0][p]), expect) < TOL_BF16
        np.testing.assert_allclose(run.lse[0][p], np.log(p + 1), rtol=TOL_F32)
    # real queries at position 0 too
    prob2 = synth.AttnProblem([L], nq, nkv, d, [q], [k], [v])
    run2 = PagedRun(prob2, page_seed=9)
    run2.prefill([(0, 64)])
    for h in range(nq):
        assert np.array_equal(run2.out[0][0, h], v[0, h // grp])


def test_repeat_bitwise():
    lens, _ = synth.ragged_lengths(8, 2048, seed=11)
    prob = _gqa(lens, seed=11)
    base = None
    for rep in range(5):
        run = PagedRun(prob, page_seed=rep)
        run.prefill([(b, L - 1) for b, L in enumerate(lens)])
        run.decode(list(range(8)))
        cur = [o.copy() for o in run.out]
        if base is None:
            base = cur
        for a, b in zip(base, cur):
            assert np.array_equal(a, b)


@pytest.mark.parametrize("B,maxlen", [(300, 600), (256, 2048), (512, 300)])
def test_decode_large_and_mixed_batches(orc, B, maxlen):
    """Decode over batches at and past the size the balanced unit list
    covers (256 sequences), with sequences from 1 to 8 splits: every decoded
    row equals the same row of a one-shot prefill.  8 q heads over 2 kv heads
    (group 4, d=128) keep the inputs small; the unit list does not depend on
    the head counts."""
    rng = synth.stream(31, "large_batch.lens")
    lens = [int(x) for x in rng.integers(2, maxlen + 1, size=B)]
    lens[0], lens[-1] = 2, maxlen  # shortest and longest in one batch
    prob = synth.attn_problem(lens, n_q=8, n_kv=2, d=128, seed=31,
                              tags=["lb%d" % i for i in range(B)])
    one = PagedRun(prob, page_seed=1)
    one.prefill([(b, L) for b, L in enumerate(lens)])
    dec = PagedRun(prob, page_seed=2)
    dec.prefill([(b, L - 2) for b, L in enumerate(lens)])
    dec.decode(list(range(B)))
    dec.decode(list(range(B)))
    for b, L in enumerate(lens):
        assert np.array_equal(dec.out[b][L - 2:], one.out[b][L - 2:]), b
        assert np.array_equal(dec.lse[b][L - 2:].view(np.uint32), one.lse[b][L - 2:].view(np.uint32)), b
    picks = [(b, lens[b] - 1) for b in (0, 1, B // 2, B - 1)]
    _parity(orc, prob, dec, picks)
