"""Shared helpers for the GPU tests: device transfer of bf16 bit patterns, the
parity metric, and a driver that runs a schedule of prefill / decode calls
over a paged key/value pool."""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

import synth

EPS = float(np.float32(1e-6))
TOL_BF16 = 2e-2   # max relative error, bf16 outputs
TOL_F32 = 1e-4    # fp32-accumulated intermediates (rstd, fp32 C, lse)


def dev():
    return torch.device("cuda:0")


def to_dev(bits: np.ndarray) -> torch.Tensor:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev())


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64(bits) -> np.ndarray:
    return synth.bf16_to_f32(bits).astype(np.float64)


def rel_err(got, ref) -> float:
    """max_i |g_i - o_i| / max(|o_i|, rms(o over the last axis)): relative error
    that stays meaningful where outputs cancel to near zero."""
    g = np.asarray(got, dtype=np.float64)
    o = np.asarray(ref, dtype=np.float64)
    if g.size == 0:
        return 0.0
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True))
    den = np.maximum(np.abs(o), np.maximum(rms, 1e-300))
    return float(np.max(np.abs(g - o) / den))


def poison_like(t: torch.Tensor) -> torch.Tensor:
    """Fill with NaN so unwritten outputs are visible."""
    return t.fill_(float("nan"))


# --------------------------------------------------------------------------- attention

class PagedRun:
    """Drives calls over one paged pool for a fixed set of sequences.

    Each call names (sequence, n_new) pairs.  prefill() sends them through
    bi_attn_prefill; decode() sends one token per named sequence through
    bi_attn_decode (or a comparator).  Outputs land in out[b][pos] as bf16 bits
    and lse[b][pos] as fp32."""

    def __init__(self, prob: synth.AttnProblem, page_seed: int = 0, extra_pages: int = 3,
                 capacities: Optional[Sequence[int]] = None):
        self.p = prob
        caps = list(capacities) if capacities is not None else list(prob.lens)
        pool = synth.page_pool(caps, prob.n_kv, prob.d, seed=page_seed, extra_pages=extra_pages)
        self.kc = to_dev(pool.k_pages)
        self.vc = to_dev(pool.v_pages)
        self.bt_host = pool.block_table
        self.bt = torch.from_numpy(pool.block_table).to(dev())
        self.cur = [0] * len(prob.lens)
        self.out = [np.full((L, prob.n_q, prob.d), 0xFFFF, dtype=np.uint16) for L in prob.lens]
        self.lse = [np.full((L, prob.n_q), np.nan, dtype=np.float32) for L in prob.lens]

    @property
    def scale(self):
        return self.p.scale

    def _rows(self, seqs):
        return torch.from_numpy(np.ascontiguousarray(self.bt_host[list(seqs)])).to(dev())

    def prefill(self, items: Sequence[Tuple[int, int]], fn=None):
        import invariant_bi_matmul_amd as bi
        fn = fn or bi.attn_prefill
        seqs = [b for b, _ in items]
        qs, ks, vs, cu, kvl = [], [], [], [0], []
        for b, n in items:
            c = self.cur[b]
            qs.append(self.p.q[b][c:c + n])
            ks.append(self.p.k[b][c:c + n])
            vs.append(self.p.v[b][c:c + n])
            cu.append(cu[-1] + n)
            kvl.append(c + n)
        q = to_dev(np.concatenate(qs))
        out = poison_like(torch.empty_like(q))
        lse = poison_like(torch.empty(q.shape[0], self.p.n_q, dtype=torch.float32, device=dev()))
        fn(q, to_dev(np.concatenate(ks)), to_dev(np.concatenate(vs)),
           torch.tensor(cu, dtype=torch.int32, device=dev()),
           torch.tensor(kvl, dtype=torch.int32, device=dev()), self._rows(seqs), self.kc, self.vc,
           self.scale, max(n for _, n in items), out=out, lse=lse)
        ob, lb = bits_of(out), lse.cpu().numpy()
        for i, (b, n) in enumerate(items):
            c = self.cur[b]
            self.out[b][c:c + n] = ob[cu[i]:cu[i] + n]
            self.lse[b][c:c + n] = lb[cu[i]:cu[i] + n]
            self.cur[b] = c + n

    def decode(self, seqs: Sequence[int], comparator: bool = False, num_splits: int = 0):
        import invariant_bi_matmul_amd as bi
        c = [self.cur[b] for b in seqs]
        q = to_dev(np.stack([self.p.q[b][c[i]] for i, b in enumerate(seqs)]))
        k = to_dev(np.stack([self.p.k[b][c[i]] for i, b in enumerate(seqs)]))
        v = to_dev(np.stack([self.p.v[b][c[i]] for i, b in enumerate(seqs)]))
        kvl = [x + 1 for x in c]
        out = poison_like(torch.empty_like(q))
        lse = poison_like(torch.empty(len(seqs), self.p.n_q, dtype=torch.float32, device=dev()))
        args = (q, k, v, torch.tensor(kvl, dtype=torch.int32, device=dev()), self._rows(seqs),
                self.kc, self.vc, self.scale, max(kvl))
        if comparator:
            bi.bix_attn_decode_splitkv(*args, num_splits=num_splits, out=out, lse=lse)
        else:
            ws = poison_like(torch.empty(bi.attn_workspace_bytes(
                bi.make_shape(len(seqs), self.p.n_q, self.p.n_kv, self.p.d, self.bt.shape[1],
                              self.kc.shape[0], self.scale), len(seqs), max(kvl)) // 4 + 4,
                dtype=torch.float32, device=dev()))
            bi.attn_decode(*args, workspace=ws, out=out, lse=lse)
        ob, lb = bits_of(out), lse.cpu().numpy()
        for i, b in enumerate(seqs):
            self.out[b][c[i]] = ob[i]
            self.lse[b][c[i]] = lb[i]
            self.cur[b] = c[i] + 1

    def run_chunked(self, chunk: int, seqs: Optional[Sequence[int]] = None):
        """Prefill every named sequence to its full length, `chunk` tokens per call."""
        seqs = list(range(len(self.p.lens))) if seqs is None else list(seqs)
        while True:
            items = [(b, min(chunk, self.p.lens[b] - self.cur[b])) for b in seqs
                     if self.cur[b] < self.p.lens[b]]
            if not items:
                break
            self.prefill(items)


def oracle_attention(orc, prob: synth.AttnProblem, picks: Sequence[Tuple[int, int]]):
    """fp64 oracle output for (sequence, position) picks -> (out [n, nq, d], lse [n, nq])."""
    k = np.concatenate(prob.k)
    v = np.concatenate(prob.v)
    q = np.stack([prob.q[b][p] for b, p in picks])
    return orc.attention(q, k, v, prob.lens, [b for b, _ in picks], [p for _, p in picks],
                         prob.scale)


def lse_err(got, ref) -> float:
    g = np.asarray(got, dtype=np.float64)
    o = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(g - o) / np.maximum(np.abs(o), 1.0))) if g.size else 0.0
