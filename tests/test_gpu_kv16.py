"""Attention over the int16 KV cache: codes and factors bit-exact against the
oracle's quantiser, outputs against fp64 attention over the dequantised
values, and the invariance contract (one-shot prefill = chunked prefill =
decode, alone or batched) on this cache too."""
import numpy as np
import pytest
import torch

import synth
from helpers import TOL_BF16, dev, rel_err
import invariant_bi_matmul_amd as bi
from oracle import kv16

pytestmark = pytest.mark.gpu


def _t(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev()).view(torch.bfloat16)


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


class Cache:
    """int16 pages + factors, pages handed out in a seeded random order."""

    def __init__(self, num_pages, nkv, d, seed=0):
        self.kc = torch.zeros(num_pages, nkv, 16, d, dtype=torch.int16, device=dev())
        self.vc = torch.zeros_like(self.kc)
        self.kf = torch.zeros(num_pages, nkv, 16, dtype=torch.float32, device=dev())
        self.vf = torch.zeros_like(self.kf)
        self.free = synth.stream(seed, "kv16.pages").permutation(num_pages).tolist()
        self.pages = {}

    def table(self, sids, lens):
        for sid, L in zip(sids, lens):
            pg = self.pages.setdefault(sid, [])
            while len(pg) * 16 < L:
                pg.append(self.free.pop())
        maxp = max(len(self.pages[s]) for s in sids)
        rows = [self.pages[s] + [self.pages[s][-1]] * (maxp - len(self.pages[s])) for s in sids]
        return torch.tensor(rows, dtype=torch.int32, device=dev())


def _seq(L, nq, nkv, d, seed, tag):
    return (synth.normal_bits((L, nq, d), 0, 1, seed, tag + ".q"),
            synth.normal_bits((L, nkv, d), 0, 1, seed, tag + ".k"),
            synth.normal_bits((L, nkv, d), 0, 1, seed, tag + ".v"))


def _prefill(cache, sids, chunks, starts, q, k, v, scale):
    """One prefill call: sequence sids[i] brings its rows starts[i] .. +chunks[i]."""
    cu = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    lens = [s + c for s, c in zip(starts, chunks)]
    bt = cache.table(sids, lens)
    rows = lambda a: np.concatenate([a[i][s:s + c] for i, (s, c) in enumerate(zip(starts, chunks))])
    return bi.attn_prefill_i16(_t(rows(q)), _t(rows(k)), _t(rows(v)),
                               torch.from_numpy(cu).to(dev()),
                               torch.tensor(lens, dtype=torch.int32, device=dev()), bt, cache.kc,
                               cache.vc, cache.kf, cache.vf, scale, max(chunks))


@pytest.mark.parametrize("nq,nkv,d,L", [(4, 2, 64, 300), (32, 8, 128, 700)])
def test_codes_and_parity(nq, nkv, d, L):
    scale = float(np.float32(1 / np.sqrt(d)))
    q, k, v = _seq(L, nq, nkv, d, 0, "kv16.p%d" % d)
    cache = Cache(64, nkv, d)
    out = _prefill(cache, [0], [L], [0], [q], [k], [v], scale)
    # the codes and factors in the pages, bit for bit
    qk, fk = kv16.quantize(k)
    qv, fv = kv16.quantize(v)
    pages = cache.pages[0]
    for j in range(0, L, 37):
        p, sl = pages[j // 16], j % 16
        assert np.array_equal(cache.kc[p, :, sl].cpu().numpy(), qk[j])
        assert np.array_equal(cache.vc[p, :, sl].cpu().numpy(), qv[j])
        assert np.array_equal(cache.kf[p, :, sl].cpu().numpy(), fk[j])
        assert np.array_equal(cache.vf[p, :, sl].cpu().numpy(), fv[j])
    ref, _ = kv16.attention(q, kv16.dequantize(qk, fk), kv16.dequantize(qv, fv), np.arange(L),
                            scale)
    assert rel_err(synth.bf16_to_f32(_bits(out)), ref) < TOL_BF16


@pytest.mark.parametrize("nq,nkv,d", [(32, 8, 128), (8, 2, 64)])
def test_chunked_prefill_and_decode_equal_one_shot(nq, nkv, d):
    L, P = 600, 540
    scale = float(np.float32(1 / np.sqrt(d)))
    q, k, v = _seq(L, nq, nkv, d, 1, "kv16.c")
    one = _bits(_prefill(Cache(64, nkv, d, 1), [0], [L], [0], [q], [k], [v], scale))
    cache = Cache(64, nkv, d, 2)
    got = []
    for s in range(0, P, 128):
        n = min(128, P - s)
        got.append(_bits(_prefill(cache, [0], [n], [s], [q], [k], [v], scale)))
    for p in range(P, L):
        bt = cache.table([0], [p + 1])
        o = bi.attn_decode_i16(_t(q[p:p + 1]), _t(k[p:p + 1]), _t(v[p:p + 1]),
                               torch.tensor([p + 1], dtype=torch.int32, device=dev()), bt,
                               cache.kc, cache.vc, cache.kf, cache.vf, scale)
        got.append(_bits(o))
    assert np.array_equal(np.concatenate(got), one)


@pytest.mark.parametrize("nb", [5, 300])
def test_decode_alone_equals_decode_in_a_batch(nb):
    """A sequence's decode row is the same alone and among nb - 1 others (300
    sequences: past the decode kernel's balanced unit list)."""
    nq, nkv, d = 32, 8, 128
    scale = float(np.float32(1 / np.sqrt(d)))
    lens = [700, 33, 1200, 257, 500]
    if nb > len(lens):
        lens += synth.stream(9, "kv16.lens").integers(2, 120, size=nb - len(lens)).tolist()
    seqs = [_seq(L, nq, nkv, d, 3, "kv16.b%d" % i) for i, L in enumerate(lens)]
    # everything but the last token of every sequence, then one decode step
    alone = Cache(512, nkv, d, 3)
    _prefill(alone, [2], [lens[2] - 1], [0], [seqs[2][0]], [seqs[2][1]], [seqs[2][2]], scale)
    batch = Cache(sum((L + 15) // 16 for L in lens) + 16, nkv, d, 4)
    n = len(lens)
    _prefill(batch, list(range(n)), [L - 1 for L in lens], [0] * n, [s[0] for s in seqs],
             [s[1] for s in seqs], [s[2] for s in seqs], scale)

    def step(cache, idx):
        last = lambda a: np.stack([a[i][lens[i] - 1] for i in idx])
        bt = cache.table(idx, [lens[i] for i in idx])
        return _bits(bi.attn_decode_i16(
            _t(last([s[0] for s in seqs])), _t(last([s[1] for s in seqs])),
            _t(last([s[2] for s in seqs])),
            torch.tensor([lens[i] for i in idx], dtype=torch.int32, device=dev()), bt, cache.kc,
            cache.vc, cache.kf, cache.vf, scale))

    a = step(alone, [2])
    b = step(batch, list(range(n)))
    assert np.array_equal(a[0], b[2])
