"""Benchmark of the batch-invariant hot path on one MI355X.

One step is one pass of the whole path over one batch of Llama-8B-shaped
synthetic input, every stage through libbi's HIP kernels:

  1. RMSNorm      x bf16 [2048, 4096] -> y                      (bi_rmsnorm)
  2. matmul       y [2048, 4096] x W bf16 [4096, 14336] -> C bf16 (bi_matmul)
  3. prefill      one sequence's 512-token chunk at positions 3584..4095 of a
                  paged cache (GQA 32/8, d=128): append + attention (bi_attn_prefill)
  4. decode       64 sequences, lengths ~U{2048..4096} (one of length 4096),
                  one new token each: append + split partials + fold (bi_attn_decode)

The headline `value` is the invariant matmul's TFLOP/s (2*M*N*K over the
matmul's average duration, from HIP events on the launch stream over the timed
steps); RMSNorm and decode-attention GB/s and the prefill TFLOP/s are in
`components`, each with its roofline fraction.  All inputs are resident in HBM
before timing starts.  Also reported: the non-invariant comparators on the same
inputs (cost of invariance), a bitwise invariance check, and the fp64 oracle
timed on the host's cores on a bounded sample of the matmul.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E
MFMA_BF16_PEAK = 2500.0   # TFLOP/s, dense bf16

M, K, N = 2048, 4096, 14336
H = 4096
NQ, NKV, D = 32, 8, 128
B_DEC, L_MAX = 64, 4096
PREFILL_CHUNK = 512


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "invariant_bi_matmul_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class Workload:
    def __init__(self, seed: int = 0):
        import numpy as np
        import torch

        import invariant_bi_matmul_amd as bi
        import synth
        self.bi, self.torch, self.np, self.synth = bi, torch, np, synth
        dev = torch.device("cuda:0")
        self.dev = dev

        def to_dev(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
                torch.bfloat16).to(dev)

        self.to_dev = to_dev
        # RMSNorm + matmul (host bits kept for the oracle sample)
        self.x_bits, self.g_bits = synth.rmsnorm_inputs(M, H, seed=seed)
        _, self.w_bits = synth.matmul_inputs(1, N, K, seed=seed)
        self.x = to_dev(self.x_bits)
        self.g = to_dev(self.g_bits)
        self.w = to_dev(self.w_bits)
        self.y = torch.empty(M, H, dtype=torch.bfloat16, device=dev)
        self.c = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        self.eps = float(np.float32(1e-6))
        # attention: 64 decoding sequences + 1 sequence in chunked prefill
        lens, self.probe = synth.ragged_lengths(B_DEC, L_MAX, seed=seed)
        self.dec_lens = lens
        self.pre_len = L_MAX
        caps = lens + [self.pre_len]
        pages = [(c + 15) // 16 for c in caps]
        self.num_pages = sum(pages) + 3
        perm = synth.stream(seed, "bench.pages").permutation(self.num_pages).astype(np.int32)
        maxp = max(pages)
        bt = np.full((len(caps), maxp), -1, dtype=np.int32)
        cur = 0
        for b, p in enumerate(pages):
            bt[b, :p] = perm[cur:cur + p]
            cur += p
        self.bt_host = bt
        self.bt_dec = torch.from_numpy(bt[:B_DEC].copy()).to(dev)
        self.bt_pre = torch.from_numpy(bt[B_DEC:].copy()).to(dev)
        shape = (self.num_pages, NKV, 16, D)
        self.kc = synth.device_normal_bf16(shape, 0.0, 1.0, seed, "bench.kpool", dev)
        self.vc = synth.device_normal_bf16(shape, 0.0, 1.0, seed, "bench.vpool", dev)
        self.scale = float(np.float32(1.0 / np.sqrt(D)))
        # decode inputs
        self.q_dec = to_dev(synth.normal_bits((B_DEC, NQ, D), 0, 1, seed, "bench.qdec"))
        self.k_dec = to_dev(synth.normal_bits((B_DEC, NKV, D), 0, 1, seed, "bench.kdec"))
        self.v_dec = to_dev(synth.normal_bits((B_DEC, NKV, D), 0, 1, seed, "bench.vdec"))
        self.kvl_dec = torch.tensor(lens, dtype=torch.int32, device=dev)
        self.out_dec = torch.empty(B_DEC, NQ, D, dtype=torch.bfloat16, device=dev)
        self.lse_dec = torch.empty(B_DEC, NQ, dtype=torch.float32, device=dev)
        ash = bi.make_shape(B_DEC, NQ, NKV, D, maxp, self.num_pages, self.scale)
        self.ws_bytes = bi.attn_workspace_bytes(ash, B_DEC, L_MAX)
        self.ws = torch.empty(self.ws_bytes // 4 + 4, dtype=torch.float32, device=dev)
        # prefill inputs: positions pre_len-512 .. pre_len-1
        T = PREFILL_CHUNK
        self.q_pre = to_dev(synth.normal_bits((T, NQ, D), 0, 1, seed, "bench.qpre"))
        self.k_pre = to_dev(synth.normal_bits((T, NKV, D), 0, 1, seed, "bench.kpre"))
        self.v_pre = to_dev(synth.normal_bits((T, NKV, D), 0, 1, seed, "bench.vpre"))
        self.cu_pre = torch.tensor([0, T], dtype=torch.int32, device=dev)
        self.kvl_pre = torch.tensor([self.pre_len], dtype=torch.int32, device=dev)
        self.out_pre = torch.empty(T, NQ, D, dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()

    # -- the four stages ------------------------------------------------------
    def rmsnorm(self):
        self.bi.rmsnorm(self.x, self.g, self.eps, out=self.y)

    def matmul(self):
        self.bi.matmul(self.y, self.w, out=self.c)

    def prefill(self):
        self.bi.attn_prefill(self.q_pre, self.k_pre, self.v_pre, self.cu_pre, self.kvl_pre,
                             self.bt_pre, self.kc, self.vc, self.scale, PREFILL_CHUNK,
                             out=self.out_pre)

    def decode(self):
        self.bi.attn_decode(self.q_dec, self.k_dec, self.v_dec, self.kvl_dec, self.bt_dec,
                            self.kc, self.vc, self.scale, L_MAX, workspace=self.ws,
                            out=self.out_dec, lse=self.lse_dec)

    STAGES = ("rmsnorm", "matmul", "prefill", "decode")

    # -- algorithmic work ------------------------------------------------------
    def work(self):
        kv_tok = sum(self.dec_lens)
        pos0 = self.pre_len - PREFILL_CHUNK
        pre_pairs = sum(p + 1 for p in range(pos0, self.pre_len))  # (query, key) pairs
        return {
            # bytes: read x, write y (2 B each), gamma once
            "rmsnorm": {"bytes": 2 * M * H * 2 + 2 * H},
            "matmul": {"flops": 2.0 * M * N * K, "bytes": 2 * (M * K + K * N + M * N)},
            # causal attention of 512 queries x 32 heads: QK^T and PV, 4*d flops per pair
            "prefill": {"flops": 4.0 * D * NQ * pre_pairs},
            # K and V of every cached position (8 kv heads, d=128, bf16) + q, out, new k/v
            "decode": {"bytes": kv_tok * NKV * D * 2 * 2 + B_DEC * NQ * D * 2 * 2
                       + B_DEC * NKV * D * 2 * 2},
        }


def time_steps(wl, steps, warmup):
    import torch
    for _ in range(warmup):
        for s in wl.STAGES:
            getattr(wl, s)()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(wl.STAGES) + 1)]
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record()
        for j, s in enumerate(wl.STAGES):
            getattr(wl, s)()
            ev[i][j + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {s: 0.0 for s in wl.STAGES}
    for i in range(steps):
        for j, s in enumerate(wl.STAGES):
            per[s] += ev[i][j].elapsed_time(ev[i][j + 1])
    return wall, {s: per[s] / steps for s in wl.STAGES}  # ms


def time_call(fn, reps=20, warmup=3):
    import torch
    for _ in range(warmup):
        fn()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps  # ms


def invariance_check(wl):
    """Bitwise: matmul rows at M=8 vs M=2048; RMSNorm rows at 8 vs 2048 rows;
    the probe sequence's decode row alone vs in the batch of 64."""
    import torch
    bi = wl.bi
    res = {}
    c8 = bi.matmul(wl.y[:8].contiguous(), wl.w)
    res["matmul"] = bool(torch.equal(c8.view(torch.int16), wl.c[:8].view(torch.int16)))
    y8 = bi.rmsnorm(wl.x[:8].contiguous(), wl.g, wl.eps)
    res["rmsnorm"] = bool(torch.equal(y8.view(torch.int16), wl.y[:8].view(torch.int16)))
    p = wl.probe
    o1 = bi.attn_decode(wl.q_dec[p:p + 1].contiguous(), wl.k_dec[p:p + 1].contiguous(),
                        wl.v_dec[p:p + 1].contiguous(), wl.kvl_dec[p:p + 1].contiguous(),
                        wl.bt_dec[p:p + 1].contiguous(), wl.kc, wl.vc, wl.scale, L_MAX)
    res["attn_decode"] = bool(torch.equal(o1[0].view(torch.int16), wl.out_dec[p].view(torch.int16)))
    torch.cuda.synchronize()
    return res


# The decoder stack's projections (Llama-8B shape, fused as the stack runs
# them): (K, N) per layer, and the lm_head once per token.
STACK_MATMULS = {"qkv": (4096, 6144), "o": (4096, 4096), "gate_up": (4096, 28672),
                 "down": (14336, 4096), "lm_head": (4096, 128256)}


def time_alternating(fns, rounds=2, reps=20, warmup=3):
    """Each call timed `rounds` times with the calls taking turns, and the best
    of each kept, so that neither side of a ratio is the one timed while the
    clock or the caches were still settling."""
    best = [None] * len(fns)
    for _ in range(rounds):
        for i, f in enumerate(fns):
            t = time_call(f, reps=reps, warmup=warmup)
            best[i] = t if best[i] is None else min(best[i], t)
    return best


def comparators(wl):
    """Invariant kernel vs its non-invariant comparator on the same inputs (ms),
    warm, timed in turns (best of two).  Matmul: the decoder stack's projection shapes at M = 1, 16, 64 (the
    decode batches) and the step's 2048 x 4096 x 14336, each beside split-K
    (bi_matmul's tile with k split to fill idle CUs) and the vendor GEMM
    (torch.matmul, not batch-invariant), and both invariant and split-K again
    with the weight in the strip layout (bi_matmul_pack_w, as the stack holds
    it); `stack_token_ms` adds up one decode token's projections (32 layers +
    lm_head) for each kernel."""
    import torch
    bi, synth, dev = wl.bi, wl.synth, wl.dev
    out = {}
    lib = bi.load()
    a_big = synth.device_normal_bf16((2048, 14336), 0.0, 1.0, 0, "cmp.a", dev)
    shapes = [("step_2048x4096x14336", 2048, 4096, 14336)]
    for m in (1, 16, 64):
        for name, (k, n) in STACK_MATMULS.items():
            shapes.append(("%s_M%d" % (name, m), m, k, n))
    most = max(lib.bix_matmul_workspace_bytes(m, n, k, 0) for _, m, k, n in shapes)
    ws = torch.empty(most // 4 + 16, dtype=torch.float32, device=dev)
    ws_cache = {}
    per_token = {m: {"invariant": 0.0, "splitk": 0.0, "vendor": 0.0, "invariant_packed": 0.0,
                     "splitk_packed": 0.0} for m in (1, 16, 64)}
    for label, m, k, n in shapes:
        if (k, n) not in ws_cache:
            ws_cache[(k, n)] = (wl.w if (k, n) == (K, N) else
                                synth.device_normal_bf16((k, n), 0.0, k ** -0.5, 0,
                                                         "cmp.w%dx%d" % (k, n), dev))
        w = ws_cache[(k, n)]
        a = a_big[:m, :k].contiguous()
        c = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
        need = lib.bix_matmul_workspace_bytes(m, n, k, 0)
        wp = bi.matmul_pack_w(w)  # the strip layout, as the stack holds its weights
        ti, tc, tv, tip, tcp = time_alternating([
            lambda: bi.matmul(a, w, out=c),
            lambda: bi.bix_matmul_splitk(a, w, out=c, workspace=ws[:need // 4 + 4]),
            lambda: torch.matmul(a, w, out=c),
            lambda: bi.matmul_packed(a, wp, out=c),
            lambda: bi.bix_matmul_splitk(a, wp, out=c, workspace=ws[:need // 4 + 4])])
        del wp
        splits = max(1, need // (4 * m * n))
        if splits == 1:
            # no CU left idle: the comparator launches the invariant kernel itself,
            # and the two timings differ only by noise (clock, order)
            ti = tc = min(ti, tc)
            tip = tcp = min(tip, tcp)
        out["matmul_" + label] = {"invariant_ms": ti, "splitk_ms": tc, "vendor_ms": tv,
                                  "invariant_packed_ms": tip, "splitk_packed_ms": tcp,
                                  "splitk_slices": splits,
                                  "invariant_over_splitk": ti / tc,
                                  "invariant_over_vendor": ti / tv,
                                  "invariant_over_splitk_packed": tip / tcp}
        if label != shapes[0][0]:
            reps = 1 if label.startswith("lm_head") else 32
            for kind, t in (("invariant", ti), ("splitk", tc), ("vendor", tv),
                            ("invariant_packed", tip), ("splitk_packed", tcp)):
                per_token[m][kind] += reps * t
    for m, r in per_token.items():
        r["invariant_over_splitk"] = r["invariant"] / r["splitk"]
        r["invariant_over_vendor"] = r["invariant"] / r["vendor"]
        r["invariant_over_splitk_packed"] = r["invariant_packed"] / r["splitk_packed"]
    out["stack_token_ms"] = per_token
    del ws, a_big, ws_cache
    for r in (1, 16, 2048):
        xr = wl.x[:r].contiguous()
        wsr = torch.empty(r * 64, dtype=torch.float32, device=dev)
        yr = torch.empty_like(xr)
        ti, tc = time_alternating([
            lambda: bi.rmsnorm(xr, wl.g, wl.eps, out=yr),
            lambda: bi.bix_rmsnorm_splitrow(xr, wl.g, wl.eps, out=yr, workspace=wsr)])
        out["rmsnorm_rows%d" % r] = {"invariant_ms": ti, "splitrow_ms": tc,
                                     "invariant_over_splitrow": ti / tc}
    for bsz in (1, 8, 64):
        sl = slice(0, bsz)
        args = (wl.q_dec[sl].contiguous(), wl.k_dec[sl].contiguous(), wl.v_dec[sl].contiguous(),
                wl.kvl_dec[sl].contiguous(), wl.bt_dec[sl].contiguous(), wl.kc, wl.vc, wl.scale,
                L_MAX)
        o = torch.empty(bsz, NQ, D, dtype=torch.bfloat16, device=dev)
        ti, tc = time_alternating([lambda: bi.attn_decode(*args, out=o),
                                   lambda: bi.bix_attn_decode_splitkv(*args, out=o)])
        out["decode_B%d_L%d" % (bsz, L_MAX)] = {"invariant_ms": ti, "splitkv_ms": tc,
                                                "invariant_over_splitkv": ti / tc}
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def _paged(wl, lens, tag):
    """A paged pool (seeded page permutation) for `lens`, drawn on the GPU."""
    import torch
    np, synth, dev = wl.np, wl.synth, wl.dev
    pages = [(l + 15) // 16 for l in lens]
    num = sum(pages) + 3
    perm = synth.stream(0, tag + ".pages").permutation(num).astype(np.int32)
    bt = np.full((len(lens), max(pages)), -1, dtype=np.int32)
    cur = 0
    for b, p in enumerate(pages):
        bt[b, :p] = perm[cur:cur + p]
        cur += p
    kc = synth.device_normal_bf16((num, NKV, 16, D), 0.0, 1.0, 0, tag + ".k", dev)
    vc = synth.device_normal_bf16((num, NKV, 16, D), 0.0, 1.0, 0, tag + ".v", dev)
    return kc, vc, torch.from_numpy(bt).to(dev)


def more_sizes(wl):
    """The same kernels at the other sizes the workload names (RMSNorm over
    16384 rows at H 4096 and 8192, decode B=16 ragged L<=32768, one-shot
    prefill of 2 x 4096), and, for context, the vendor GEMM (torch.matmul,
    not batch-invariant) at the step's matmul shape.  Warm timings."""
    import torch
    bi, synth, dev = wl.bi, wl.synth, wl.dev
    out = {}
    for h in (4096, 8192):
        x = synth.device_normal_bf16((16384, h), 0.0, 1.0, 0, "bench.rms16k.x%d" % h, dev)
        g = synth.device_normal_bf16((h,), 1.0, 0.1, 0, "bench.rms16k.g%d" % h, dev)
        y = torch.empty_like(x)
        ms = time_call(lambda: bi.rmsnorm(x, g, wl.eps, out=y))
        gbs = (2 * 16384 * h * 2 + 2 * h) / ms / 1e6
        out["rmsnorm_R16384_H%d" % h] = {"ms": ms, "GB/s": gbs, "hbm_frac": gbs / HBM_PEAK_GBS}
        del x, y
    lens, _ = synth.ragged_lengths(16, 32768, seed=0)
    kc, vc, bt = _paged(wl, lens, "bench.dec32k")
    q = synth.device_normal_bf16((16, NQ, D), 0.0, 1.0, 0, "bench.dec32k.q", dev)
    kn = synth.device_normal_bf16((16, NKV, D), 0.0, 1.0, 0, "bench.dec32k.kn", dev)
    vn = synth.device_normal_bf16((16, NKV, D), 0.0, 1.0, 0, "bench.dec32k.vn", dev)
    kvl = torch.tensor(lens, dtype=torch.int32, device=dev)
    o = torch.empty(16, NQ, D, dtype=torch.bfloat16, device=dev)
    ms = time_call(lambda: bi.attn_decode(q, kn, vn, kvl, bt, kc, vc, wl.scale, 32768, out=o))
    by = sum(lens) * NKV * D * 2 * 2 + 16 * NQ * D * 2 * 2 + 16 * NKV * D * 2 * 2
    out["decode_B16_L32768"] = {"ms": ms, "GB/s": by / ms / 1e6,
                                "hbm_frac": by / ms / 1e6 / HBM_PEAK_GBS}
    del kc, vc
    L = 4096
    kc, vc, bt = _paged(wl, [L, L], "bench.pre2x4k")
    q = synth.device_normal_bf16((2 * L, NQ, D), 0.0, 1.0, 0, "bench.pre2x4k.q", dev)
    kn = synth.device_normal_bf16((2 * L, NKV, D), 0.0, 1.0, 0, "bench.pre2x4k.kn", dev)
    vn = synth.device_normal_bf16((2 * L, NKV, D), 0.0, 1.0, 0, "bench.pre2x4k.vn", dev)
    cu = torch.tensor([0, L, 2 * L], dtype=torch.int32, device=dev)
    kvl = torch.tensor([L, L], dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    ms = time_call(lambda: bi.attn_prefill(q, kn, vn, cu, kvl, bt, kc, vc, wl.scale, L, out=o),
                   reps=5)
    fl = 4.0 * D * NQ * 2 * sum(p + 1 for p in range(L))
    out["prefill_2x4096_one_shot"] = {"ms": ms, "TFLOP/s": fl / ms / 1e9,
                                      "mfma_frac": fl / ms / 1e9 / MFMA_BF16_PEAK}
    del kc, vc, q, o
    cv = torch.empty_like(wl.c)
    tv = time_call(lambda: torch.matmul(wl.y, wl.w, out=cv))
    ti = time_call(lambda: bi.matmul(wl.y, wl.w, out=wl.c))
    out["vendor_gemm_M%d_N%d_K%d" % (M, N, K)] = {
        "torch_matmul_ms": tv, "torch_matmul_TFLOP/s": 2.0 * M * N * K / tv / 1e9,
        "invariant_ms": ti, "invariant_over_vendor": ti / tv}
    # the int16 KV cache (codes + per-(token, kv head) factors) on the step's
    # attention workloads: the same pages and block tables, random codes
    shape = (wl.num_pages, NKV, 16, D)
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    kc16 = torch.randint(-32767, 32768, shape, dtype=torch.int16, device=dev, generator=g)
    vc16 = torch.randint(-32767, 32768, shape, dtype=torch.int16, device=dev, generator=g)
    kf = torch.rand(shape[:3], dtype=torch.float32, device=dev, generator=g) * 1e-4
    vf = torch.rand(shape[:3], dtype=torch.float32, device=dev, generator=g) * 1e-4
    od = torch.empty_like(wl.out_dec)
    op = torch.empty_like(wl.out_pre)
    td = time_call(lambda: bi.attn_decode_i16(wl.q_dec, wl.k_dec, wl.v_dec, wl.kvl_dec, wl.bt_dec,
                                              kc16, vc16, kf, vf, wl.scale, out=od))
    tp = time_call(lambda: bi.attn_prefill_i16(wl.q_pre, wl.k_pre, wl.v_pre, wl.cu_pre,
                                               wl.kvl_pre, wl.bt_pre, kc16, vc16, kf, vf,
                                               wl.scale, PREFILL_CHUNK, out=op))
    w = wl.work()
    kv_tok = sum(wl.dec_lens)
    dec_bytes = w["decode"]["bytes"] + kv_tok * NKV * 4 * 2  # + the K and V factors
    out["int16_kv"] = {
        "decode_B%d_L%d" % (B_DEC, L_MAX): {"ms": td, "GB/s": dec_bytes / td / 1e6,
                                            "hbm_frac": dec_bytes / td / 1e6 / HBM_PEAK_GBS,
                                            "over_bf16_decode": td / time_call(wl.decode)},
        "prefill_chunk%d_at%d" % (PREFILL_CHUNK, L_MAX): {
            "ms": tp, "TFLOP/s": w["prefill"]["flops"] / tp / 1e9,
            "over_bf16_prefill": tp / time_call(wl.prefill)}}
    del kc16, vc16, kf, vf
    # error-compensated matmul (fp32 operands as hi/lo bf16 pairs, three
    # products in one fixed order) at the step's shape: cost against bi_matmul
    a32 = wl.y.float()
    w3 = bi.matmul_ec_pack_w(wl.w.float())
    c32 = torch.empty(M, N, dtype=torch.float32, device=dev)
    ws = torch.empty(M * 3 * K, dtype=torch.bfloat16, device=dev)
    te = time_call(lambda: bi.matmul_ec(a32, w3, out=c32, workspace=ws))
    out["matmul_ec_M%d_N%d_K%d" % (M, N, K)] = {
        "ms": te, "effective_TFLOP/s": 2.0 * M * N * K / te / 1e9,
        "mfma_TFLOP/s": 3 * 2.0 * M * N * K / te / 1e9, "over_invariant_bf16": te / ti}
    del a32, w3, c32, ws
    torch.cuda.synchronize()
    return out


def time_rotating(fns, reps):
    """Average ms per call over `reps` calls cycling through `fns` (each one a
    different buffer set, so the working set stays out of the caches)."""
    import torch
    for f in fns:
        f()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for i in range(reps):
        fns[i % len(fns)]()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def time_graph(fns, reps):
    """Average ms per call of the same rotation replayed from one captured HIP
    graph: the launches leave the host at once, so a short kernel is timed
    without Python's per-call overhead.  None if capture fails."""
    import torch
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for f in fns:
                f()
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(reps):
                fns[i % len(fns)]()
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        del g
        return a.elapsed_time(b) / reps
    except Exception as e:  # capture is a measurement aid, never a failure
        log("bench: graph capture failed: %s" % e)
        return None


ROTATE_BYTES = 512 << 20   # twice the 256 MiB MALL
CUS = 256
MFMA_FLOPS_PER_CU_CLK = 4096   # dense bf16: 2.5 PFLOP/s = 256 CUs x 4096 x 2.4 GHz


def ceilings():
    """Measured ceilings beside the datasheet peaks: a 4 GiB device copy (read +
    write), a 4 GiB read-only stream through LDS (bix_read_stream, the decode
    kernel's way of reading), and an MFMA-only
    register loop (bix_mfma_loop), whose rate over 4096 flop per CU per clock
    gives the clock the chip holds under matrix load."""
    import torch
    import invariant_bi_matmul_amd as bi
    n = 1 << 30
    src = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    ms = time_call(lambda: dst.copy_(src), reps=5, warmup=1)
    out = {"copy_4GiB": {"GB/s": 2 * 4 * n / ms / 1e6, "ms": ms,
                         "kernel": "torch copy_ (read 4 GiB + write 4 GiB)"}}
    del dst
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    best = None
    for wg in (256, 512, 1024):
        ms = time_call(lambda: bi.bix_read_stream(src, wg, sink), reps=5, warmup=1)
        gbs = 4 * n / ms / 1e6
        if best is None or gbs > best["GB/s"]:
            best = {"GB/s": gbs, "ms": ms, "workgroups": wg}
    out["read_4GiB"] = best
    del src
    fsink = torch.zeros(4, dtype=torch.float32, device="cuda")
    iters = 20000
    # fixed operands, then operands that change from one MFMA to the next (as
    # in a matmul): the second shows the clock the chip holds under the
    # matrix pipe's real power draw
    for key, varied in (("mfma_bf16_loop", False), ("mfma_bf16_loop_varied", True)):
        best = None
        for wg in (CUS * 4, CUS * 8):
            fl = 4.0 * 4 * 32768 * iters * wg
            ms = time_call(lambda: bi.bix_mfma_loop(iters, wg, fsink, varied=varied), reps=5,
                           warmup=1)
            tf = fl / ms / 1e9
            if best is None or tf > best["TFLOP/s"]:
                best = {"TFLOP/s": tf, "ms": ms, "workgroups": wg, "waves_per_simd": wg // CUS,
                        "implied_clock_GHz": tf * 1e12 / (CUS * MFMA_FLOPS_PER_CU_CLK) / 1e9}
        out[key] = best
    torch.cuda.synchronize()
    return out


def _grid_fill(tiles):
    """Fraction of CU-slots busy when `tiles` workgroups (one per CU at a
    time) run in ceil(tiles / 256) rounds."""
    rounds = -(-tiles // CUS)
    return tiles / (rounds * CUS)


def sweeps(wl, parts=("matmul", "rmsnorm", "decode", "prefill")):
    """The configurations' sizes, each timed over rotating buffer sets of at
    least 512 MiB so that every launch reads from HBM, not the MALL.

    matmul: M in {1,2,7,16,64,256,512,2048}, N in {4096, 14336}, K=4096:
    TFLOP/s, fraction of the bf16 peak, of the roofline min(peak, AI x 8 TB/s)
    and the grid-fill ceiling of the tile bi_matmul picks; beside it the vendor
    GEMM (torch.matmul, not batch-invariant) on the same buffers and
    bi_matmul_packed on the same weights in the strip layout (packed_ms).  RMSNorm: R in
    {1..16384 powers of two, 3, 7, 1000, 16383}, H in {4096, 8192}.  Decode:
    L in {512, 4096, 32768} x B in {1..64}, lengths ragged U{L/2..L} with one
    probe at L, shuffled 16-token pages.  Prefill: one sequence of L tokens,
    one-shot against 512-token chunks (and whether they agree bit for bit).
    Matmul, RMSNorm and decode are also timed replayed from a captured HIP
    graph (graph_ms), which removes the host's per-call launch cost."""
    import torch
    bi, synth, dev, np = wl.bi, wl.synth, wl.dev, wl.np
    out = {"matmul": {}, "rmsnorm": {}, "decode": {}, "prefill": {}}
    a_full = wl.y
    bi.rmsnorm(wl.x, wl.g, wl.eps, out=wl.y)
    for n in (4096, 14336) if "matmul" in parts else ():
        log("sweep: matmul N=%d" % n)
        wbytes = K * n * 2
        sets = max(1, -(-ROTATE_BYTES // wbytes))
        ws = [synth.device_normal_bf16((K, n), 0.0, 0.125, 0, "sweep.w%d.%d" % (n, i), dev)
              for i in range(sets)]
        wps = [bi.matmul_pack_w(w) for w in ws]  # the same weights in the strip layout
        for m in (1, 2, 7, 16, 64, 256, 512, 2048):
            a = a_full[:m].contiguous()
            cs = [torch.empty(m, n, dtype=torch.bfloat16, device=dev) for _ in range(sets)]
            fns = [(lambda w=w, c=c: bi.matmul(a, w, out=c)) for w, c in zip(ws, cs)]
            ms = time_rotating(fns, max(40, 2 * sets))
            gms = time_graph(fns, max(40, 2 * sets))
            vfns = [(lambda w=w, c=c: torch.matmul(a, w, out=c)) for w, c in zip(ws, cs)]
            vms = time_rotating(vfns, max(40, 2 * sets))
            pfns = [(lambda w=w, c=c: bi.matmul_packed(a, w, out=c)) for w, c in zip(wps, cs)]
            pms = time_rotating(pfns, max(40, 2 * sets))
            flops = 2.0 * m * n * K
            by = 2.0 * (m * K + K * n + m * n)
            tf = flops / ms / 1e9
            roof = min(MFMA_BF16_PEAK, flops / by * HBM_PEAK_GBS / 1e3)
            tm, tn, wgs = bi.matmul_tile(m, n)
            tiles = -(-m // tm) * -(-n // tn)
            out["matmul"]["M%d_N%d" % (m, n)] = {
                "ms": ms, "TFLOP/s": tf, "mfma_frac": tf / MFMA_BF16_PEAK,
                "roofline_TFLOP/s": roof, "roofline_frac": tf / roof,
                "GB/s": by / ms / 1e6, "tile": "%dx%d" % (tm, tn), "tiles": tiles,
                "workgroups": wgs, "grid_fill_ceiling": _grid_fill(tiles),
                "vendor_ms": vms, "invariant_over_vendor": ms / vms, "graph_ms": gms,
                "packed_ms": pms, "packed_roofline_frac": flops / pms / 1e9 / roof}
            del cs
        del ws, wps
    for h in (4096, 8192) if "rmsnorm" in parts else ():
        log("sweep: rmsnorm H=%d" % h)
        rows_big = ROTATE_BYTES // (2 * h)
        xb = synth.device_normal_bf16((rows_big, h), 0.0, 1.0, 0, "sweep.rms%d" % h, dev)
        yb = torch.empty_like(xb)
        g = synth.device_normal_bf16((h,), 1.0, 0.1, 0, "sweep.rmsg%d" % h, dev)
        for r in sorted({1 << i for i in range(15)} | {3, 7, 1000, 16383}):
            sets = max(1, min(256, rows_big // r))
            fns = [(lambda i=i: bi.rmsnorm(xb[i * r:(i + 1) * r], g, wl.eps,
                                           out=yb[i * r:(i + 1) * r])) for i in range(sets)]
            ms = time_rotating(fns, max(20, sets))
            gms = time_graph(fns, max(20, sets))
            by = 4.0 * h * r + 2 * h
            out["rmsnorm"]["R%d_H%d" % (r, h)] = {"ms": ms, "GB/s": by / ms / 1e6,
                                                  "hbm_frac": by / ms / 1e6 / HBM_PEAK_GBS,
                                                  "graph_ms": gms,
                                                  "graph_GB/s": by / gms / 1e6 if gms else None}
        del xb, yb
    for L in (512, 4096, 32768) if "decode" in parts else ():
        log("sweep: decode L=%d" % L)
        for bsz in (1, 2, 4, 8, 16, 32, 64):
            lens, _ = synth.ragged_lengths(bsz, L, seed=0)
            pages = [(l + 15) // 16 for l in lens]
            set_bytes = sum(lens) * NKV * D * 2 * 2
            sets = max(1, min(64, -(-ROTATE_BYTES // set_bytes)))
            num = sets * sum(pages) + 3
            perm = synth.stream(0, "sweep.dec.%d.%d" % (bsz, L)).permutation(num).astype(np.int32)
            kc = synth.device_normal_bf16((num, NKV, 16, D), 0.0, 1.0, 0, "sweep.dk", dev)
            vc = synth.device_normal_bf16((num, NKV, 16, D), 0.0, 1.0, 0, "sweep.dv", dev)
            bts = []
            cur = 0
            for _ in range(sets):
                bt = np.full((bsz, max(pages)), -1, dtype=np.int32)
                for b, p in enumerate(pages):
                    bt[b, :p] = perm[cur:cur + p]
                    cur += p
                bts.append(torch.from_numpy(bt).to(dev))
            q = synth.device_normal_bf16((bsz, NQ, D), 0.0, 1.0, 0, "sweep.dq", dev)
            kn = synth.device_normal_bf16((bsz, NKV, D), 0.0, 1.0, 0, "sweep.dkn", dev)
            vn = synth.device_normal_bf16((bsz, NKV, D), 0.0, 1.0, 0, "sweep.dvn", dev)
            kvl = torch.tensor(lens, dtype=torch.int32, device=dev)
            o = torch.empty(bsz, NQ, D, dtype=torch.bfloat16, device=dev)
            ash = bi.make_shape(bsz, NQ, NKV, D, max(pages), num, wl.scale)
            wsp = torch.empty(bi.attn_workspace_bytes(ash, bsz, L) // 4 + 4, dtype=torch.float32,
                              device=dev)
            fns = [(lambda bt=bt: bi.attn_decode(q, kn, vn, kvl, bt, kc, vc, wl.scale, L,
                                                 workspace=wsp, out=o)) for bt in bts]
            ms = time_rotating(fns, max(20, sets))
            gms = time_graph(fns, max(20, sets))
            by = set_bytes + bsz * NQ * D * 2 * 2 + bsz * NKV * D * 2 * 2
            out["decode"]["B%d_L%d" % (bsz, L)] = {"ms": ms, "GB/s": by / ms / 1e6,
                                                   "hbm_frac": by / ms / 1e6 / HBM_PEAK_GBS,
                                                   "kv_tokens": sum(lens), "graph_ms": gms,
                                                   "graph_GB/s": by / gms / 1e6 if gms else None}
            del kc, vc, bts
    for L in (512, 4096, 32768) if "prefill" in parts else ():
        log("sweep: prefill L=%d" % L)
        kc, vc, bt = _paged(wl, [L], "sweep.pre%d" % L)
        q = synth.device_normal_bf16((L, NQ, D), 0.0, 1.0, 0, "sweep.pq%d" % L, dev)
        kn = synth.device_normal_bf16((L, NKV, D), 0.0, 1.0, 0, "sweep.pk%d" % L, dev)
        vn = synth.device_normal_bf16((L, NKV, D), 0.0, 1.0, 0, "sweep.pv%d" % L, dev)
        one = torch.empty_like(q)
        chk = torch.empty_like(q)
        cu_one = torch.tensor([0, L], dtype=torch.int32, device=dev)
        kvl_one = torch.tensor([L], dtype=torch.int32, device=dev)
        C = PREFILL_CHUNK
        cu_c = torch.tensor([0, C], dtype=torch.int32, device=dev)
        kvls = [torch.tensor([s + C], dtype=torch.int32, device=dev) for s in range(0, L, C)]

        def chunked():
            for i, s in enumerate(range(0, L, C)):
                bi.attn_prefill(q[s:s + C], kn[s:s + C], vn[s:s + C], cu_c, kvls[i], bt, kc, vc,
                                wl.scale, C, out=chk[s:s + C])

        reps = 3 if L > 4096 else 10
        t1 = time_call(lambda: bi.attn_prefill(q, kn, vn, cu_one, kvl_one, bt, kc, vc, wl.scale,
                                               L, out=one), reps=reps, warmup=1)
        tc = time_call(chunked, reps=reps, warmup=1)
        fl = 8192.0 * L * (L + 1)
        out["prefill"]["L%d" % L] = {
            "one_shot_ms": t1, "one_shot_TFLOP/s": fl / t1 / 1e9,
            "one_shot_mfma_frac": fl / t1 / 1e9 / MFMA_BF16_PEAK,
            "chunked512_ms": tc, "chunked512_TFLOP/s": fl / tc / 1e9,
            "chunked_bitwise_equal_one_shot": bool(torch.equal(one.view(torch.int16),
                                                               chk.view(torch.int16)))}
        del kc, vc, q, kn, vn, one, chk
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _timed(run, units, target_s, max_n=None):
    """Grow n until run(n) takes a quarter of target_s, then time run(n)
    scaled to about target_s seconds (n at most max_n).  Returns (n, units(n)
    per second, seconds)."""
    cap = (lambda v: v) if max_n is None else (lambda v: min(v, max_n))
    n = 1
    while True:
        t0 = time.perf_counter()
        run(n)
        dt = time.perf_counter() - t0
        if dt >= target_s / 4 or n == cap(n + 1):
            break
        n = cap(n * 8 if dt < 1e-3 else int(n * min(8.0, target_s / 2 / dt)) + 1)
    n = cap(max(n, int(n * target_s / dt)))
    t0 = time.perf_counter()
    run(n)
    dt = time.perf_counter() - t0
    return n, units(n) / dt, dt


def cpu_oracle(wl, target_s=3.0):
    """The oracle on the host, on all cores and on one, in the GPU side's
    units: the matmul (TFLOP/s over rows of A x the full W), RMSNorm (GB/s over
    rows of x), decode attention (GB/s over sequences of the decode batch,
    keys and values gathered from the paged pool) and the prefill chunk
    (TFLOP/s over its queries, each against its own causal prefix)."""
    import numpy as np
    import oracle
    torch = wl.torch
    oracle.build(force=False)
    a_bits = wl.y.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    x_rows = np.tile(wl.x_bits, (4, 1))
    # the decode batch's keys and values, unpaged, and its queries
    bt = wl.bt_host
    kc = wl.kc.view(torch.int16).cpu().numpy().view(np.uint16)
    vc = wl.vc.view(torch.int16).cpu().numpy().view(np.uint16)
    qd = wl.q_dec.view(torch.int16).cpu().numpy().view(np.uint16)

    def unpage(pool, b):
        L = wl.dec_lens[b]
        p = bt[b, :(L + 15) // 16]
        return np.ascontiguousarray(pool[p].transpose(0, 2, 1, 3).reshape(-1, NKV, D)[:L])

    lens = wl.dec_lens
    k_all = np.concatenate([unpage(kc, b) for b in range(B_DEC)])
    v_all = np.concatenate([unpage(vc, b) for b in range(B_DEC)])
    off = np.concatenate([[0], np.cumsum(lens)])

    def decode(n):
        # the first n sequences of the batch: their keys are a prefix of k_all
        oracle.attention(qd[:n], k_all[:off[n]], v_all[:off[n]], lens[:n], list(range(n)),
                         [L - 1 for L in lens[:n]], wl.scale, threads=threads)

    def rmsnorm(n):
        # n rows, in calls over the 8192 rows at hand
        for s in range(0, n, x_rows.shape[0]):
            oracle.rmsnorm(x_rows[:min(n - s, x_rows.shape[0])], wl.g_bits, wl.eps,
                           threads=threads)

    def decode_seqs(n):
        # n sequences, in passes over the 64 of the decode batch
        for s in range(0, n, B_DEC):
            decode(min(n - s, B_DEC))

    kv_bytes = lambda n: sum(wl.dec_lens[i % B_DEC] for i in range(n)) * NKV * D * 4 / 1e9

    # the prefill chunk: its sequence's keys and values (the chunk's own rows
    # are in the pool once a step has run) and its queries at positions
    # pre_len - 512 .. pre_len - 1
    Lp = wl.pre_len
    pos0 = Lp - PREFILL_CHUNK
    pages_pre = bt[B_DEC, :(Lp + 15) // 16]
    k_pre = np.ascontiguousarray(kc[pages_pre].transpose(0, 2, 1, 3).reshape(-1, NKV, D)[:Lp])
    v_pre = np.ascontiguousarray(vc[pages_pre].transpose(0, 2, 1, 3).reshape(-1, NKV, D)[:Lp])
    q_pre = wl.q_pre.view(torch.int16).cpu().numpy().view(np.uint16)

    def prefill(n):
        # the chunk's first n queries, in passes over the chunk
        for s in range(0, n, PREFILL_CHUNK):
            m = min(n - s, PREFILL_CHUNK)
            oracle.attention(q_pre[:m], k_pre, v_pre, [Lp], [0] * m, list(range(pos0, pos0 + m)),
                             wl.scale, threads=threads)

    pre_flops = lambda n: sum(4.0 * D * NQ * (pos0 + i % PREFILL_CHUNK + 1)
                              for i in range(n)) / 1e12
    out = {"cores": oracle.default_threads(), "model": _cpu_model(), "kind": "oracle"}
    for label, threads in (("all_cores", oracle.default_threads()), ("one_core", 1)):
        r = {}
        n, v, dt = _timed(lambda n: oracle.matmul(a_bits, wl.w_bits, rows=range(n),
                                                  threads=threads),
                          lambda n: 2.0 * n * N * K / 1e12, target_s, M)
        r["matmul_TFLOP/s"] = {"value": v, "rows": n, "s": dt}
        n, v, dt = _timed(rmsnorm, lambda n: 4.0 * H * n / 1e9, target_s)
        r["rmsnorm_GB/s"] = {"value": v, "rows": n, "s": dt}
        n, v, dt = _timed(decode_seqs, kv_bytes, target_s)
        r["decode_GB/s"] = {"value": v, "sequences": n, "s": dt}
        n, v, dt = _timed(prefill, pre_flops, target_s)
        r["prefill_TFLOP/s"] = {"value": v, "queries": n, "s": dt}
        out[label] = r
    return out


def cpu_baseline(wl, target_s=12.0):
    """The fp64 oracle, as it stands, on a bounded sample of the step's matmul:
    rows of A (the RMSNorm output) times the full W, timed on this host."""
    import numpy as np
    import oracle
    oracle.build(force=False)
    a_bits = wl.y.detach().view(wl.torch.int16).cpu().numpy().view(np.uint16)
    threads = oracle.default_threads()
    rows, v, dt = _timed(lambda n: oracle.matmul(a_bits, wl.w_bits, rows=range(n),
                                                 threads=threads),
                         lambda n: 2.0 * n * N * K / 1e12, target_s, M)
    return {"value": v, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d rows of the [%d,%d]x[%d,%d] matmul, fp64, %.1f s" %
                      (rows, M, M, K, K, N, dt)}


def traffic_for(kernel_file):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    rec = t.get(kernel_file)
    if not rec or rec.get("source_sha") != source_sha(kernel_file, "common.h"):
        return None
    return rec.get("bytes_per_launch")


def calibrate_copy(nbytes=1 << 30):
    """A plain device-to-device copy of known size, for scaling the FETCH_SIZE /
    WRITE_SIZE counters (run under rocprofv3 --pmc)."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": nbytes, "launches": 3}))


def e2e_llama8b(steps: int = 128, calls: int = 30):
    """The whole stack end to end: a Llama-3-8B-shaped dense decoder (32 layers,
    hidden 4096, GQA 32/8, SwiGLU 14336, vocab 128256, random-init weights) run
    on the library's kernels.  A 256-token random prompt is decoded greedily
    for ``steps`` tokens alone and among 63 other random prompts (lengths
    U{64..512}); its tokens and logits are compared bit for bit.  Then, as the
    news.hada.io page's GPT-4 experiment counted the distinct outputs of 30
    repeated calls at temperature 0 with 128 tokens, the probe is decoded in
    ``calls`` calls, each among a different random set of companions (batch
    sizes drawn from 1..64, the probe at a random place), and its distinct
    token sequences are counted.  The same is done with the non-invariant
    comparator kernels.  Decode steps are replayed from a captured HIP graph
    (about 400 library calls per step); the prefill calls are eager.  Wall
    times include the prefill and the host's per-step bookkeeping."""
    import torch
    import synth
    from invariant_bi_matmul_amd.model import Decoder, LlamaConfig
    cfg = LlamaConfig()
    w = synth.llama_weights(cfg.hidden, cfg.layers, cfg.n_q, cfg.n_kv, cfg.head_dim, cfg.ffn,
                            cfg.vocab, seed=0)
    probe = synth.token_ids(256, cfg.vocab, 0, "e2e.probe")
    lens = synth.stream(0, "e2e.lens").integers(64, 513, size=63).tolist()
    others = [(i + 1, synth.token_ids(L, cfg.vocab, 0, "e2e.c%d" % i)) for i, L in enumerate(lens)]
    cap = 64 * (512 + steps) + 64
    rng = synth.stream(0, "e2e.calls")
    plan = []
    for _ in range(calls):
        n = int(rng.choice([1, 2, 4, 8, 16, 32, 48, 64]))
        comp = [others[i] for i in rng.permutation(63)[:n - 1]]
        at = int(rng.integers(0, n))
        plan.append(comp[:at] + [(0, probe)] + comp[at:])

    def batch_of(n):
        b = dict(others[:(n - 1) // 2])
        b[0] = probe
        b.update(others[(n - 1) // 2:n - 1])
        return b

    def differs(a, b):
        return next((i for i, (x, y) in enumerate(zip(a, b)) if x != y), None)

    out = {"config": {"layers": cfg.layers, "hidden": cfg.hidden, "n_q": cfg.n_q,
                      "n_kv": cfg.n_kv, "ffn": cfg.ffn, "vocab": cfg.vocab,
                      "rope_theta": cfg.rope_theta, "prompt": 256, "companions": 63,
                      "steps": steps, "calls": calls,
                      "call_batch_sizes": [len(b) for b in plan]}}
    for name, comp in (("invariant", False), ("comparator", True)):
        dec = Decoder(cfg, w, max_tokens=cap, comparator=comp)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        a_tok, a_log = dec.generate({0: probe}, steps, keep_logits=[0])
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        b_tok, b_log = dec.generate(batch_of(64), steps, keep_logits=[0])
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        same = [torch.equal(x.view(torch.int32), y.view(torch.int32))
                for x, y in zip(a_log[0], b_log[0])]
        uniq = set()
        for batch in plan:
            uniq.add(tuple(dec.generate(dict(batch), steps)[0][0]))
        torch.cuda.synchronize()
        out[name] = {"alone_s": t1 - t0, "batched64_s": t2 - t1,
                     "batched64_tokens_per_s": 64 * steps / (t2 - t1),
                     "tokens_equal": a_tok[0] == b_tok[0],
                     "logits_bitwise_equal": all(same),
                     "first_differing_token": differs(a_tok[0], b_tok[0]),
                     "first_differing_logits_step": next((i for i, s in enumerate(same)
                                                          if not s), None),
                     "unique_outputs_over_%d_calls" % calls: len(uniq),
                     "calls_s": time.perf_counter() - t2}
        del dec, a_log, b_log
        torch.cuda.empty_cache()
    return out


METRIC = "invariant matmul TFLOP/s + RMSNorm/attn GB/s (% roofline), bitwise row-invariance"
WORKLOAD = ("batch-invariant hot path step: RMSNorm [2048,4096] -> matmul [2048,4096]x[4096,14336]"
            " -> attention prefill chunk 512 @ 4096 + decode B=64 ragged L<=4096, GQA 32/8, "
            "d=128, 16-token pages")


def _round(v, sig=4):
    """Floats to `sig` significant digits, recursively (keeps the line short)."""
    if isinstance(v, float):
        return float("%.*g" % (sig, v)) if v == v else None
    if isinstance(v, dict):
        return {k: _round(x, sig) for k, x in v.items()}
    if isinstance(v, (list, tuple)):
        return [_round(x, sig) for x in v]
    return v


def _summary(extras):
    """The extras that fit on the headline line: the invariance verdicts, each
    comparator's time ratio and the end-to-end stack's verdicts and rates."""
    out = {}
    inv = extras.get("invariance_bitwise")
    if isinstance(inv, dict):
        out["invariance_bitwise"] = inv
    coi = extras.get("cost_of_invariance")
    if isinstance(coi, dict) and "error" not in coi:
        keep = ("matmul_step", "rmsnorm", "decode")
        out["cost_of_invariance"] = {
            k: {r: x for r, x in v.items() if r.startswith("invariant_over")}
            for k, v in coi.items() if isinstance(v, dict) and k.startswith(keep)}
        tok = coi.get("stack_token_ms")
        if isinstance(tok, dict):
            out["cost_of_invariance"]["stack_token_matmuls"] = {
                "M%s" % m: {r: x for r, x in v.items() if r.startswith("invariant_over")}
                for m, v in tok.items()}
    e2e = extras.get("e2e_llama8b")
    if isinstance(e2e, dict) and "error" not in e2e:
        keep = ("tokens_equal", "logits_bitwise_equal", "batched64_tokens_per_s", "alone_s")
        out["e2e_llama8b"] = {
            name: {k: v for k, v in r.items() if k in keep or k.startswith("unique_outputs")}
            for name, r in e2e.items() if name != "config" and isinstance(r, dict)}
    for name, r in extras.items():
        if isinstance(r, dict) and "error" in r:
            out.setdefault("failed_extras", []).append(name)
    return out


def headline(steps, warmup, ms_step, tflops, comp, cpu, traffic, extras, extras_path):
    """The one JSON line bench.py prints: the step's headline, its roofline
    and host baseline, the four stages and a summary of the extras (a few KB
    at most; the full record goes to `extras_path`)."""
    keep = ("ms", "graph_ms", "GB/s", "TFLOP/s", "hbm_frac", "mfma_frac", "graph_frac")
    line = {
        "metric": METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Llama-8B-shaped tensors, random-init weights)",
        "config": {"workload": WORKLOAD, "M": M, "K": K, "N": N, "decode_batch": B_DEC,
                   "max_kv_len": L_MAX, "prefill_chunk": PREFILL_CHUNK},
        "roofline": {"bound": "mfma", "kernel": "bi_matmul_kernel", "achieved": tflops,
                     "peak": MFMA_BF16_PEAK, "unit": "TFLOP/s", "frac": tflops / MFMA_BF16_PEAK,
                     "traffic": traffic},
        "cpu_baseline": cpu,
        "components": {k: {f: v for f, v in c.items() if f in keep} for k, c in comp.items()},
    }
    line = _round(line)
    line["value"] = tflops
    line["ms_per_step"] = ms_step
    line.update(_round(_summary(extras)))
    line["extras_file"] = extras_path
    return line


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the comparator timings and the invariance check")
    ap.add_argument("--no-e2e", action="store_true",
                    help="skip the end-to-end Llama-8B-shaped invariance run")
    ap.add_argument("--no-sweeps", action="store_true",
                    help="skip the size sweeps and the measured ceilings")
    ap.add_argument("--only", choices=("sweeps", "ceilings"),
                    help="run only the size sweeps or the ceilings and print them")
    ap.add_argument("--sweep-parts", default="matmul,rmsnorm,decode,prefill",
                    help="with --only sweeps: which sweeps, comma-separated")
    ap.add_argument("--stage", choices=("rmsnorm", "matmul", "prefill", "decode"),
                    help="run one pass of the step, then only this stage, --warmup + --steps "
                         "times (for profiler passes), and print its average time")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--extras-out", default=os.path.join("gpurun_out", "bench_extras.json"),
                    help="where the full record (sweeps, ceilings, comparators, e2e, oracle "
                         "timings) is written; the printed line keeps a summary")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(see the sharding notes in DESIGN.md); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.only == "ceilings":
        print(json.dumps({"ceilings": ceilings()}))
        return
    log("bench: generating inputs")
    wl = Workload()
    if args.only == "sweeps":
        print(json.dumps({"sweeps": sweeps(wl, tuple(args.sweep_parts.split(",")))}))
        return
    if args.stage:
        # one pass of the whole step first, so that the stage's inputs hold
        # the step's values (the matmul reads the RMSNorm output; MFMA power,
        # and so the clock, depends on the operand values)
        for s in wl.STAGES:
            getattr(wl, s)()
        fn = getattr(wl, args.stage)
        ms = time_call(fn, reps=args.steps, warmup=args.warmup)
        print(json.dumps({"stage": args.stage, "calls": args.steps, "ms": ms}))
        return
    log("bench: warmup %d, timing %d steps" % (args.warmup, args.steps))
    torch.cuda.synchronize()
    wall, per = time_steps(wl, args.steps, args.warmup)
    ms_step = wall * 1e3 / args.steps
    w = wl.work()
    mm_ms = per["matmul"]
    tflops = w["matmul"]["flops"] / (mm_ms * 1e-3) / 1e12
    comp = {
        "rmsnorm": {"ms": per["rmsnorm"], "GB/s": w["rmsnorm"]["bytes"] / per["rmsnorm"] / 1e6},
        "matmul": {"ms": mm_ms, "TFLOP/s": tflops},
        "attn_prefill": {"ms": per["prefill"],
                         "TFLOP/s": w["prefill"]["flops"] / per["prefill"] / 1e9},
        "attn_decode": {"ms": per["decode"], "GB/s": w["decode"]["bytes"] / per["decode"] / 1e6},
    }
    # the same stages replayed from a captured graph: the kernels' own time,
    # without the events' and the host's per-launch gaps (short stages only
    # differ)
    for name, key, unit, work in (("rmsnorm", "rmsnorm", "GB/s", w["rmsnorm"]["bytes"] / 1e6),
                                  ("matmul", "matmul", "TFLOP/s", w["matmul"]["flops"] / 1e9),
                                  ("prefill", "attn_prefill", "TFLOP/s", w["prefill"]["flops"] / 1e9),
                                  ("decode", "attn_decode", "GB/s", w["decode"]["bytes"] / 1e6)):
        gms = time_graph([getattr(wl, name)], 20)
        comp[key]["graph_ms"] = gms
        comp[key]["graph_" + unit] = work / gms if gms else None
    comp["rmsnorm"]["hbm_frac"] = comp["rmsnorm"]["GB/s"] / HBM_PEAK_GBS
    comp["matmul"]["mfma_frac"] = tflops / MFMA_BF16_PEAK
    comp["attn_prefill"]["mfma_frac"] = comp["attn_prefill"]["TFLOP/s"] / MFMA_BF16_PEAK
    comp["attn_decode"]["hbm_frac"] = comp["attn_decode"]["GB/s"] / HBM_PEAK_GBS
    # the same fractions from the graph replays (the kernels' own time)
    for key, unit, peak in (("rmsnorm", "GB/s", HBM_PEAK_GBS), ("matmul", "TFLOP/s", MFMA_BF16_PEAK),
                            ("attn_prefill", "TFLOP/s", MFMA_BF16_PEAK),
                            ("attn_decode", "GB/s", HBM_PEAK_GBS)):
        g = comp[key].get("graph_" + unit)
        comp[key]["graph_frac"] = g / peak if g else None
    extras = {}

    def extra(name, fn):
        """Run one optional measurement; a failure is recorded in the line
        instead of losing the step's numbers."""
        try:
            extras[name] = fn()
        except Exception as e:  # noqa: BLE001 - reported, never hidden
            log("bench: %s failed: %r" % (name, e))
            extras[name] = {"error": repr(e)}

    if not args.no_extras:
        log("bench: invariance check and comparators")
        extra("invariance_bitwise", lambda: invariance_check(wl))
        extra("cost_of_invariance", lambda: comparators(wl))
        log("bench: other sizes")
        extra("more_sizes", lambda: more_sizes(wl))
        if not args.no_sweeps:
            log("bench: measured ceilings")
            extra("ceilings", ceilings)
            c = extras["ceilings"]
            if "error" not in c:
                extras["vs_measured_ceilings"] = {
                    "matmul_over_mfma_loop": tflops / c["mfma_bf16_loop"]["TFLOP/s"],
                    "matmul_over_mfma_loop_varied": tflops / c["mfma_bf16_loop_varied"]["TFLOP/s"],
                    "decode_over_read_stream": comp["attn_decode"]["GB/s"] / c["read_4GiB"]["GB/s"],
                    "rmsnorm_over_copy": comp["rmsnorm"]["GB/s"] / c["copy_4GiB"]["GB/s"]}
            log("bench: size sweeps")
            extra("sweeps", lambda: sweeps(wl))
        if not args.no_e2e:
            log("bench: end-to-end Llama-8B-shaped stack, alone vs 63 companions")
            extra("e2e_llama8b", e2e_llama8b)
    cpu = None
    if not args.no_cpu_baseline:
        log("bench: oracle on the host")
        cpu = cpu_baseline(wl)
        if not args.no_extras:
            log("bench: oracle on all cores and on one")
            extra("cpu_oracle", lambda: cpu_oracle(wl))
    traffic = traffic_for("matmul.hip")
    line = headline(args.steps, args.warmup, ms_step, tflops, comp, cpu, traffic, extras,
                    args.extras_out)
    if args.extras_out:
        full = dict(line)
        full["components"] = comp
        full.update(extras)
        try:
            os.makedirs(os.path.dirname(os.path.abspath(args.extras_out)), exist_ok=True)
            with open(args.extras_out, "w") as f:
                json.dump(full, f)
            log("bench: full record in %s" % args.extras_out)
        except OSError as e:
            log("bench: could not write %s: %r" % (args.extras_out, e))
    print(json.dumps(line))

if __name__ == "__main__":
    main()
