"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This module holds no arithmetic of the method: it draws random numbers, rounds
them to bf16 bit patterns (round to nearest, ties to even), and lays tokens out
in a paged key/value pool.  Both sides of every parity check receive exactly
the arrays made here; neither side's results ever flow back into it.

Recipe (Llama-8B-shaped synthetic data; no dataset or trained weights):

* streams: ``numpy.random.default_rng(SeedSequence(seed, spawn_key=(tag,)))``,
  one independent stream per named tensor, seed 0 unless a test says otherwise;
  values are drawn in float32, then rounded to bf16.
* N(mu, sigma): the second parameter is the standard deviation.
* RMSNorm rows: N(0, 1) with each element independently, with probability
  0.01, replaced by a draw from N(0, 30); gamma ~ N(1, 0.1).
* matmul: A ~ N(0, 1); W ~ N(0, 1/sqrt(K)) (1/16 at K=256, 1/64 at K=4096).
* attention: Q, K, V ~ N(0, 1); 16-token pages; physical pages are a seeded
  random permutation of the pool; ragged lengths ~ U{L/2 .. L} with a probe
  sequence of length L at a random batch index.
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

BF16_NAN_POISON = 0x7FC0  # quiet NaN as bf16 bits


def stream(seed: int, tag: str) -> np.random.Generator:
    """An independent generator for one named tensor."""
    key = zlib.crc32(tag.encode("utf-8"))
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(key,)))


def bf16_bits(x) -> np.ndarray:
    """float32 values -> bf16 bit patterns, round to nearest even (NaN kept NaN)."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = ((u[nan] >> 16).astype(np.uint16) | 0x0040)
    return out


def bf16_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact), for building test inputs only."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


def normal_bits(shape, mean: float, std: float, seed: int, tag: str) -> np.ndarray:
    g = stream(seed, tag)
    return bf16_bits(g.normal(mean, std, size=shape).astype(np.float32))


def rmsnorm_inputs(rows: int, hidden: int, seed: int = 0, outliers: bool = True):
    """x bits [rows, hidden] and gamma bits [hidden].  Row i is the same for
    every row count (prefix-stable), which the row-invariance checks rely on."""
    g = stream(seed, "rms.x.%d" % hidden)
    x = g.normal(0.0, 1.0, size=(rows, hidden)).astype(np.float32)
    if outliers:
        # Mask and replacement values come from streams of their own, drawn for
        # every element, so the first r rows are the same for any row count.
        mask = stream(seed, "rms.outmask.%d" % hidden).random(size=(rows, hidden)) < 0.01
        big = stream(seed, "rms.outval.%d" % hidden).normal(0.0, 30.0, size=(rows, hidden))
        x = np.where(mask, big.astype(np.float32), x)
    gamma = normal_bits((hidden,), 1.0, 0.1, seed, "rms.gamma.%d" % hidden)
    return bf16_bits(x), gamma


def matmul_inputs(m: int, n: int, k: int, seed: int = 0):
    """A bits [m, k] ~ N(0,1) and W bits [k, n] ~ N(0, 1/sqrt(k)).

    A's rows come from one stream per k, so A[:m] is the same for every m (the
    row-i-fixed-across-M property of the workload)."""
    a = normal_bits((m, k), 0.0, 1.0, seed, "mm.a.%d" % k)
    w = normal_bits((k, n), 0.0, 1.0 / np.sqrt(k), seed, "mm.w.%d.%d" % (k, n))
    return a, w


def ragged_lengths(batch: int, max_len: int, seed: int = 0, probe_len: Optional[int] = None):
    """Lengths ~ U{max_len//2 .. max_len}; one probe of length probe_len (default
    max_len) at a random index.  Returns (lengths, probe_index)."""
    g = stream(seed, "attn.lens.%d.%d" % (batch, max_len))
    lo = max(1, max_len // 2)
    lens = g.integers(lo, max_len + 1, size=batch)
    probe = int(g.integers(0, batch))
    lens[probe] = max_len if probe_len is None else probe_len
    return [int(v) for v in lens], probe


@dataclass
class PagedKV:
    """A paged key/value pool plus its block table.

    k_pages, v_pages: bf16 bits [num_pages, n_kv, page_size, d]
    block_table: int32 [batch, max_pages_per_seq]; entry i of row b is the
    physical page holding positions 16*i .. 16*i+15 of sequence b.  Unused
    entries hold -1 (and are never read for positions < the sequence length).
    """
    k_pages: np.ndarray
    v_pages: np.ndarray
    block_table: np.ndarray
    page_size: int
    capacity: List[int] = field(default_factory=list)


def page_pool(capacities: Sequence[int], n_kv: int, d: int, page_size: int = 16,
              seed: int = 0, extra_pages: int = 3, poison: bool = True) -> PagedKV:
    """Allocate pages for sequences of the given token capacities, assigning
    physical pages by a seeded random permutation.  Pool contents are poison
    (bf16 NaN) so a read of an unwritten slot shows up."""
    need = [(c + page_size - 1) // page_size for c in capacities]
    total = int(sum(need)) + extra_pages
    maxp = max(need) if need else 0
    perm = stream(seed, "attn.pages.%d" % total).permutation(total).astype(np.int32)
    bt = np.full((len(capacities), max(maxp, 1)), -1, dtype=np.int32)
    cur = 0
    for b, np_ in enumerate(need):
        bt[b, :np_] = perm[cur:cur + np_]
        cur += np_
    fill = BF16_NAN_POISON if poison else 0
    kp = np.full((total, n_kv, page_size, d), fill, dtype=np.uint16)
    vp = np.full((total, n_kv, page_size, d), fill, dtype=np.uint16)
    return PagedKV(kp, vp, bt, page_size, list(capacities))


def scatter_tokens(pool: PagedKV, b: int, start: int, k_bits: np.ndarray, v_bits: np.ndarray):
    """Place tokens start..start+n-1 of sequence b (k/v bits [n, n_kv, d]) into
    the pool.  Used to pre-fill a cache as test input."""
    n = k_bits.shape[0]
    ps = pool.page_size
    for i in range(n):
        p = start + i
        page = pool.block_table[b, p // ps]
        pool.k_pages[page, :, p % ps, :] = k_bits[i]
        pool.v_pages[page, :, p % ps, :] = v_bits[i]


@dataclass
class AttnProblem:
    """Logical per-sequence Q/K/V for B sequences (bf16 bits).

    q[b]: [L_b, n_q, d], k[b], v[b]: [L_b, n_kv, d] -- row j is position j."""
    lens: List[int]
    n_q: int
    n_kv: int
    d: int
    q: List[np.ndarray]
    k: List[np.ndarray]
    v: List[np.ndarray]

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / np.sqrt(self.d)))


def attn_seq(L: int, n_q: int, n_kv: int, d: int, seed: int = 0, tag: str = "s"):
    """One sequence's (q, k, v) bits, [L, n_q, d] and [L, n_kv, d] x2.  Depends
    on (seed, tag, shape) only, so a sequence is the same whatever its batch."""
    q = normal_bits((L, n_q, d), 0.0, 1.0, seed, "attn.q.%s.%d.%d" % (tag, n_q, d))
    k = normal_bits((L, n_kv, d), 0.0, 1.0, seed, "attn.k.%s.%d.%d" % (tag, n_kv, d))
    v = normal_bits((L, n_kv, d), 0.0, 1.0, seed, "attn.v.%s.%d.%d" % (tag, n_kv, d))
    return q, k, v


def attn_problem(lens: Sequence[int], n_q: int, n_kv: int, d: int, seed: int = 0,
                 tags: Optional[Sequence[str]] = None) -> AttnProblem:
    """Q/K/V ~ N(0,1) for each sequence; sequence b uses tag tags[b] (default
    "s<b>"), so giving a sequence the same tag reproduces it at any batch index
    and beside any companions."""
    if tags is None:
        tags = ["s%d" % b for b in range(len(lens))]
    qs, ks, vs = [], [], []
    for L, t in zip(lens, tags):
        q, k, v = attn_seq(L, n_q, n_kv, d, seed, t)
        qs.append(q)
        ks.append(k)
        vs.append(v)
    return AttnProblem(list(lens), n_q, n_kv, d, qs, ks, vs)


def device_normal_bf16(shape, mean: float, std: float, seed: int, tag: str, device="cuda"):
    """Large N(mean, std) bf16 tensors drawn directly on the GPU with torch's
    seeded Philox generator (used for the benchmark's key/value pool, where a
    host-side draw would dominate set-up time).  Rounded to bf16 by torch's
    round-to-nearest-even conversion."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed((seed << 32) ^ zlib.crc32(tag.encode("utf-8")))
    t = torch.empty(shape, dtype=torch.float32, device=device)
    t.normal_(mean, std, generator=g)
    return t.to(torch.bfloat16)


def llama_weights(hidden: int, layers: int, n_q: int, n_kv: int, head_dim: int, ffn: int,
                  vocab: int, seed: int = 0, device="cuda"):
    """Random-init weights of a Llama-style stack, drawn on the GPU (see
    ``device_normal_bf16``): every projection [in, out] ~ N(0, 1/sqrt(in)),
    the embedding table ~ N(0, 1), RMSNorm gammas ~ N(1, 0.1).  No trained
    weights exist here; this only gives the stack realistic magnitudes."""
    def mat(shape, tag):
        return device_normal_bf16(shape, 0.0, 1.0 / np.sqrt(shape[0]), seed, tag, device)

    def gamma(tag):
        return device_normal_bf16((hidden,), 1.0, 0.1, seed, tag, device)

    qd, kvd = n_q * head_dim, n_kv * head_dim
    out = {"embed": device_normal_bf16((vocab, hidden), 0.0, 1.0, seed, "llama.embed", device),
           "final_norm": gamma("llama.final_norm"),
           "lm_head": mat((hidden, vocab), "llama.lm_head"),
           "layers": []}
    for i in range(layers):
        t = "llama.%d." % i
        out["layers"].append({
            "attn_norm": gamma(t + "attn_norm"), "wq": mat((hidden, qd), t + "wq"),
            "wk": mat((hidden, kvd), t + "wk"), "wv": mat((hidden, kvd), t + "wv"),
            "wo": mat((qd, hidden), t + "wo"), "mlp_norm": gamma(t + "mlp_norm"),
            "w_gate": mat((hidden, ffn), t + "w_gate"), "w_up": mat((hidden, ffn), t + "w_up"),
            "w_down": mat((ffn, hidden), t + "w_down")})
    return out


def llama_weights_host(hidden: int, layers: int, n_q: int, n_kv: int, head_dim: int, ffn: int,
                       vocab: int, seed: int = 0, fp32: bool = False) -> dict:
    """The same kind of random-init weights drawn on the host (numpy), for
    stacks small enough to check against the oracle: bf16 bit patterns
    (uint16) everywhere, or, with ``fp32``, the projections and the lm_head as
    unrounded float32 values (the embedding table and gammas stay bf16).
    Projections [in, out] ~ N(0, 1/sqrt(in)), embedding ~ N(0, 1), gammas
    ~ N(1, 0.1)."""
    def mat(shape, tag):
        x = stream(seed, tag).standard_normal(shape, dtype=np.float32) / np.float32(
            np.sqrt(shape[0]))
        return x if fp32 else bf16_bits(x)

    def gamma(tag):
        return normal_bits((hidden,), 1.0, 0.1, seed, tag)

    qd, kvd = n_q * head_dim, n_kv * head_dim
    out = {"embed": normal_bits((vocab, hidden), 0.0, 1.0, seed, "llama.h.embed"),
           "final_norm": gamma("llama.h.final_norm"),
           "lm_head": mat((hidden, vocab), "llama.h.lm_head"),
           "layers": []}
    for i in range(layers):
        t = "llama.h.%d." % i
        out["layers"].append({
            "attn_norm": gamma(t + "attn_norm"), "wq": mat((hidden, qd), t + "wq"),
            "wk": mat((hidden, kvd), t + "wk"), "wv": mat((hidden, kvd), t + "wv"),
            "wo": mat((qd, hidden), t + "wo"), "mlp_norm": gamma(t + "mlp_norm"),
            "w_gate": mat((hidden, ffn), t + "w_gate"), "w_up": mat((hidden, ffn), t + "w_up"),
            "w_down": mat((ffn, hidden), t + "w_down")})
    return out


def token_ids(n: int, vocab: int, seed: int, tag: str) -> List[int]:
    """n random token ids, uniform over the vocabulary."""
    return stream(seed, tag).integers(0, vocab, size=n).tolist()
