// Paged split-KV attention: append, split partials, fixed-order fold.
//
// Follows the Attention row of the approach table in "Defeating
// Nondeterminism in LLM Inference" (mobiles-han.blogspot.com summary):
//   * one unified layout -- a call first appends its new keys/values to the
//     paged pool (kv_append_kernel); attention then reads the pool only, so a
//     token's keys take the same path whether they arrived in this call or
//     long ago;
//   * fixed-size splits -- keys are cut at absolute multiples of 256.  The
//     partial of one split for one query column is computed by ONE device
//     function (split_partial), and partials are folded left in ascending
//     split order by ONE device function (fold_step).  Prefill folds in
//     registers; decode writes partials to a workspace and a second kernel
//     folds them; both call the same functions with the same operands, so a
//     token's output row has the same bits either way.
//
// Work unit: one wave64 computes the partial of one split for a block of 16
// query columns (GQA: the columns are (position, head-of-group) pairs sharing
// one kv head) with v_mfma_f32_16x16x32_bf16:
//   S^T = K Q^T   (A = 16 keys x 32 dims, B = Q^T in registers)
//   O^T = V^T P^T (A = 16 dims x 32 keys, B = P^T straight from registers)
// Keys of a 32-key chunk are permuted onto MFMA rows so that each lane's
// accumulator holds the 8 consecutive keys it needs as the P^T operand; V is
// transposed in registers, lane r owning dims DB*r .. DB*r+DB-1 (DB = d/16).
// Masked keys (beyond the query position) get logit -inf and weight exactly
// 0, and their addresses are clamped to a written position, so they add
// exact zeros; chunks wholly beyond every column's position are skipped,
// which is therefore exact too.
//
// bix_attn_decode_splitkv_* is the comparator from the problem column of the
// same row: the key range of each sequence is cut into a number of splits
// chosen from the batch, so split boundaries move with the batch.
#include <limits.h>

#include "common.h"
#include "kernels.h"

namespace bi {
namespace {

constexpr float kLn2 = 0.693147180559945309f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// One step of the left fold:  m' = max(m, ms); l = l e^(m-m') + ls e^(ms-m'),
// o = o e^(m-m') + os e^(ms-m') (base-2 logits, so e^ is exp2).
struct FoldCoef {
  float a, b, m;
};
__device__ __forceinline__ FoldCoef fold_coef(float m, float ms) {
  const float mn = fmaxf(m, ms);
  return FoldCoef{fast_exp2(m - mn), fast_exp2(ms - mn), mn};
}
__device__ __forceinline__ float fold_apply(float x, float xs, const FoldCoef& f) {
  return x * f.a + xs * f.b;
}
// Natural-log lse from base-2 max and sum.
__device__ __forceinline__ float lse_of(float m2, float l) { return (m2 + fast_log2(l)) * kLn2; }

template <int D>
struct KV {
  static constexpr int DS = D / 32;  // 32-wide MFMA k-steps over the head dim
  static constexpr int DB = D / 16;  // O^T row blocks; lane owns DB consecutive dims
};

// Address of position `pos` of one sequence / kv head in a paged pool.
template <int D>
__device__ __forceinline__ const uint16_t* kv_row(const uint16_t* pool, const int32_t* bt_row,
                                                  int nkv, int g, int pos) {
  const int page = bt_row[pos >> 4];
  return pool + ((((int64_t)page * nkv + g) << 4) + (pos & 15)) * D;
}

// Partial of keys key0 .. key0 + 32*nchunks - 1 for this wave's 16 columns.
// Lane l (r = l%16, q = l/16) owns column r, whose query sits at position
// pcol; key j is valid iff j <= pcol and j < key_end.  Addresses of keys at
// or beyond `written` (a count of written positions) are clamped to
// written-1.  Returns m (base-2 max logit, -inf if nothing valid), l, and o
// (lane holds dims DB*(4q+t)+i in o[i][t]).
template <int D>
__device__ __forceinline__ void split_partial(const uint16_t* __restrict__ kc,
                                              const uint16_t* __restrict__ vc,
                                              const int32_t* __restrict__ bt_row, int nkv, int g,
                                              int written, int key0, int nchunks, int key_end,
                                              const bf16x8 (&qf)[KV<D>::DS], int pcol, float c2,
                                              float& m_out, float& l_out,
                                              f32x4 (&o)[KV<D>::DB]) {
  constexpr int DS = KV<D>::DS, DB = KV<D>::DB;
  const int lane = threadIdx.x & (kWave - 1);
  const int r = lane & 15, q = lane >> 4;
  const int last = written - 1;

  float z[8][8];  // z[c][j]: key key0 + 32c + 8q + j, column r
  // ---- S^T = K Q^T, chunk by chunk ----
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    if (c < nchunks) {
      f32x4 acc[2] = {f32x4{}, f32x4{}};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int key = key0 + 32 * c + 8 * (r >> 2) + 4 * h + (r & 3);
        const uint16_t* kp = kv_row<D>(kc, bt_row, nkv, g, min(key, last)) + 8 * q;
#pragma unroll
        for (int t = 0; t < DS; ++t) {
          const u32x4 a = *(const u32x4*)(kp + 32 * t);
          acc[h] = mfma16(as_bf16x8(a), qf[t], acc[h]);
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = key0 + 32 * c + 8 * q + 4 * h + i;
          const bool ok = key <= pcol && key < key_end;
          z[c][4 * h + i] = ok ? acc[h][i] * c2 : -INFINITY;
        }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) z[c][j] = -INFINITY;
    }
  }
  // ---- max, exponentials, sum: fixed order (chunks, then keys, then lanes) ----
  float m = -INFINITY;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, z[c][j]);
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  float l = 0.0f;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float e = z[c][j] == -INFINITY ? 0.0f : fast_exp2(z[c][j] - m);
      z[c][j] = e;
      l = l + e;
    }
  l = l + __shfl_xor(l, 16);
  l = l + __shfl_xor(l, 32);

  // ---- O^T = V^T P^T ----
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = f32x4{};
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    if (c < nchunks) {
      const u32x4 pw = u32x4{pack_bf16x2(z[c][0], z[c][1]), pack_bf16x2(z[c][2], z[c][3]),
                             pack_bf16x2(z[c][4], z[c][5]), pack_bf16x2(z[c][6], z[c][7])};
      const bf16x8 pf = as_bf16x8(pw);
      if constexpr (DB == 8) {
        u32x4 vr[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int key = key0 + 32 * c + 8 * q + j;
          vr[j] = *(const u32x4*)(kv_row<D>(vc, bt_row, nkv, g, min(key, last)) + DB * r);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int w = i >> 1;
          u32x4 va;
          if (i & 1)
            va = u32x4{pack_hi(vr[0][w], vr[1][w]), pack_hi(vr[2][w], vr[3][w]),
                       pack_hi(vr[4][w], vr[5][w]), pack_hi(vr[6][w], vr[7][w])};
          else
            va = u32x4{pack_lo(vr[0][w], vr[1][w]), pack_lo(vr[2][w], vr[3][w]),
                       pack_lo(vr[4][w], vr[5][w]), pack_lo(vr[6][w], vr[7][w])};
          o[i] = mfma16(as_bf16x8(va), pf, o[i]);
        }
      } else {
        static_assert(DB == 4, "head_dim 64 or 128");
        u32x2 vr[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int key = key0 + 32 * c + 8 * q + j;
          vr[j] = *(const u32x2*)(kv_row<D>(vc, bt_row, nkv, g, min(key, last)) + DB * r);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int w = i >> 1;
          u32x4 va;
          if (i & 1)
            va = u32x4{pack_hi(vr[0][w], vr[1][w]), pack_hi(vr[2][w], vr[3][w]),
                       pack_hi(vr[4][w], vr[5][w]), pack_hi(vr[6][w], vr[7][w])};
          else
            va = u32x4{pack_lo(vr[0][w], vr[1][w]), pack_lo(vr[2][w], vr[3][w]),
                       pack_lo(vr[4][w], vr[5][w]), pack_lo(vr[6][w], vr[7][w])};
          o[i] = mfma16(as_bf16x8(va), pf, o[i]);
        }
      }
    }
  }
  m_out = m;
  l_out = l;
}

// Q^T operand for d-step t: dims 32t + 8q .. +7 of this lane's query row.
template <int D>
__device__ __forceinline__ void load_q(const uint16_t* qrow, bool live, bf16x8 (&qf)[KV<D>::DS]) {
  const int q = (threadIdx.x & (kWave - 1)) >> 4;
#pragma unroll
  for (int t = 0; t < KV<D>::DS; ++t) {
    const u32x4 v = live ? *(const u32x4*)(qrow + 32 * t + 8 * q) : u32x4{0u, 0u, 0u, 0u};
    qf[t] = as_bf16x8(v);
  }
}

// ---- append ------------------------------------------------------------------
// blockIdx.y = sequence, blockIdx.x = token index within this call's tokens
// of that sequence.  cu_q == nullptr means one token per sequence (decode).
template <int D>
__global__ __launch_bounds__(128) void kv_append_kernel(const uint16_t* __restrict__ k_new,
                                                        const uint16_t* __restrict__ v_new,
                                                        const int32_t* __restrict__ cu_q,
                                                        const int32_t* __restrict__ kv_len,
                                                        const int32_t* __restrict__ bt,
                                                        uint16_t* __restrict__ kc,
                                                        uint16_t* __restrict__ vc, int nkv,
                                                        int max_pages) {
  const int b = blockIdx.y;
  const int i = blockIdx.x;
  int tok0 = b, nb = 1;
  if (cu_q != nullptr) {
    tok0 = cu_q[b];
    nb = cu_q[b + 1] - tok0;
  }
  if (i >= nb) return;
  const int pos = kv_len[b] - nb + i;
  const int64_t tok = tok0 + i;
  const int page = bt[(int64_t)b * max_pages + (pos >> 4)];
  const int slot = pos & 15;
  const int vecs = nkv * (D / 8);
  for (int idx = threadIdx.x; idx < vecs; idx += blockDim.x) {
    const int g = idx / (D / 8), e = (idx % (D / 8)) * 8;
    const int64_t src = (tok * nkv + g) * D + e;
    const int64_t dst = ((((int64_t)page * nkv + g) << 4) + slot) * D + e;
    *(u32x4*)(kc + dst) = *(const u32x4*)(k_new + src);
    *(u32x4*)(vc + dst) = *(const u32x4*)(v_new + src);
  }
}

// ---- decode ------------------------------------------------------------------
// One wave per (sequence b, kv head g, split s); 4 waves per workgroup.
// Workspace record per (b, q head, s): o[D], m, l  (fp32).
template <int D>
__global__ __launch_bounds__(256) void bi_attn_decode_partial_kernel(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ kv_len,
    const int32_t* __restrict__ bt, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, float* __restrict__ ws, int B, int nq, int nkv, int max_pages,
    int smax, float c2) {
  constexpr int DB = KV<D>::DB;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int s = (int)(u % smax);
  const int64_t rest = u / smax;
  const int g = (int)(rest % nkv);
  const int b = (int)(rest / nkv);
  if (b >= B) return;
  const int L = kv_len[b];
  const int key0 = s * kSplit;
  if (key0 >= L) return;
  const int group = nq / nkv;
  const int col = lane & 15;
  const bool live = col < group;
  const int hq = g * group + (live ? col : 0);
  bf16x8 qf[KV<D>::DS];
  load_q<D>(q + ((int64_t)b * nq + hq) * D, live, qf);
  const int pcol = L - 1;
  const int nch = min(8, (L - key0 + 31) / 32);
  float m, l;
  f32x4 o[DB];
  split_partial<D>(kc, vc, bt + (int64_t)b * max_pages, nkv, g, L, key0, nch, INT_MAX, qf, pcol,
                   c2, m, l, o);
  if (live) {
    float* rec = ws + (((int64_t)b * nq + hq) * smax + s) * (D + 2);
    const int qq = lane >> 4;
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t) rec[DB * (4 * qq + t) + i] = o[i][t];
    if (qq == 0) {
      rec[D] = m;
      rec[D + 1] = l;
    }
  }
}

// Fold the splits of one (sequence, q head) left in ascending order.
// Thread d owns output dim d.  nsplit_of: splits actually present.
template <int D>
__global__ __launch_bounds__(D) void bi_attn_combine_kernel(const float* __restrict__ ws,
                                                            const int32_t* __restrict__ kv_len,
                                                            uint16_t* __restrict__ out,
                                                            float* __restrict__ lse, int nq,
                                                            int smax, int split_len) {
  const int64_t bh = blockIdx.x;
  const int b = (int)(bh / nq);
  const int d = threadIdx.x;
  const int L = kv_len[b];
  const int ns = min(smax, (L + split_len - 1) / split_len);
  const float* rec = ws + bh * smax * (D + 2);
  float m = rec[D], l = rec[D + 1], o = rec[d];
  for (int s = 1; s < ns; ++s) {
    const float* rs = rec + (int64_t)s * (D + 2);
    const FoldCoef f = fold_coef(m, rs[D]);
    l = fold_apply(l, rs[D + 1], f);
    o = fold_apply(o, rs[d], f);
    m = f.m;
  }
  out[bh * D + d] = (uint16_t)f32_to_bf16(o / l);
  if (lse != nullptr && d == 0) lse[bh] = lse_of(m, l);
}

// ---- prefill -----------------------------------------------------------------
// Grid (query tiles, kv heads, sequences); 4 waves per workgroup, each wave a
// block of 16/group positions x group heads.  Tiles run latest-first.
template <int D>
__global__ __launch_bounds__(256) void bi_attn_prefill_kernel(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ kv_len, const int32_t* __restrict__ bt,
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc, uint16_t* __restrict__ out,
    float* __restrict__ lse, int nq, int nkv, int max_pages, float c2) {
  constexpr int DB = KV<D>::DB;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int b = blockIdx.z, g = blockIdx.y;
  const int tile = (int)(gridDim.x - 1 - blockIdx.x);
  const int group = nq / nkv;
  const int ppw = 16 / group;  // positions per wave
  const int tok0 = cu_q[b];
  const int nb = cu_q[b + 1] - tok0;
  const int i0 = (tile * 4 + wave) * ppw;
  if (i0 >= nb) return;
  const int L = kv_len[b];
  const int start = L - nb;
  const int col = lane & 15;
  const int pi = i0 + col / group;
  const bool live = pi < nb;
  const int hq = g * group + col % group;
  const int64_t tok = tok0 + min(pi, nb - 1);
  bf16x8 qf[KV<D>::DS];
  load_q<D>(q + (tok * nq + hq) * D, live, qf);
  const int pcol = live ? start + pi : -1;
  const int pmax = start + min(i0 + ppw, nb) - 1;
  const int32_t* bt_row = bt + (int64_t)b * max_pages;

  float M = -INFINITY, Lsum = 0.0f;
  f32x4 O[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) O[i] = f32x4{};
  const int nsplit = pmax / kSplit + 1;
  for (int s = 0; s < nsplit; ++s) {
    const int key0 = s * kSplit;
    const int nch = min(8, (pmax - key0 + 32) / 32);
    float ms, ls;
    f32x4 os[DB];
    split_partial<D>(kc, vc, bt_row, nkv, g, L, key0, nch, INT_MAX, qf, pcol, c2, ms, ls, os);
    if (key0 <= pcol) {
      if (s == 0) {
        M = ms;
        Lsum = ls;
#pragma unroll
        for (int i = 0; i < DB; ++i) O[i] = os[i];
      } else {
        const FoldCoef f = fold_coef(M, ms);
        Lsum = fold_apply(Lsum, ls, f);
#pragma unroll
        for (int i = 0; i < DB; ++i)
#pragma unroll
          for (int t = 0; t < 4; ++t) O[i][t] = fold_apply(O[i][t], os[i][t], f);
        M = f.m;
      }
    }
  }
  if (live) {
    const int64_t orow = (tok * nq + hq) * D;
    const int qq = lane >> 4;
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        out[orow + DB * (4 * qq + t) + i] = (uint16_t)f32_to_bf16(O[i][t] / Lsum);
    if (lse != nullptr && qq == 0) lse[tok * nq + hq] = lse_of(M, Lsum);
  }
}

// ---- comparator: split count chosen from the batch ---------------------------
// Split p of a sequence covers keys [p*len, (p+1)*len); inside it, blocks of
// 256 keys counted from the split's start are folded in registers.
template <int D>
__global__ __launch_bounds__(256) void bix_attn_decode_splitkv_kernel(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ kv_len,
    const int32_t* __restrict__ bt, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, float* __restrict__ ws, int B, int nq, int nkv, int max_pages,
    int nsplit, int split_len, float c2) {
  constexpr int DB = KV<D>::DB;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int sp = (int)(u % nsplit);
  const int64_t rest = u / nsplit;
  const int g = (int)(rest % nkv);
  const int b = (int)(rest / nkv);
  if (b >= B) return;
  const int L = kv_len[b];
  const int k_begin = sp * split_len;
  if (k_begin >= L) return;
  const int k_end = min(L, k_begin + split_len);
  const int group = nq / nkv;
  const int col = lane & 15;
  const bool live = col < group;
  const int hq = g * group + (live ? col : 0);
  bf16x8 qf[KV<D>::DS];
  load_q<D>(q + ((int64_t)b * nq + hq) * D, live, qf);
  float M = -INFINITY, Lsum = 0.0f;
  f32x4 O[DB];
  for (int key0 = k_begin; key0 < k_end; key0 += kSplit) {
    const int nch = min(8, (k_end - key0 + 31) / 32);
    float ms, ls;
    f32x4 os[DB];
    split_partial<D>(kc, vc, bt + (int64_t)b * max_pages, nkv, g, L, key0, nch, k_end, qf, L - 1,
                     c2, ms, ls, os);
    if (key0 == k_begin) {
      M = ms;
      Lsum = ls;
#pragma unroll
      for (int i = 0; i < DB; ++i) O[i] = os[i];
    } else {
      const FoldCoef f = fold_coef(M, ms);
      Lsum = fold_apply(Lsum, ls, f);
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int t = 0; t < 4; ++t) O[i][t] = fold_apply(O[i][t], os[i][t], f);
      M = f.m;
    }
  }
  if (live) {
    float* rec = ws + (((int64_t)b * nq + hq) * nsplit + sp) * (D + 2);
    const int qq = lane >> 4;
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t) rec[DB * (4 * qq + t) + i] = O[i][t];
    if (qq == 0) {
      rec[D] = M;
      rec[D + 1] = Lsum;
    }
  }
}

float base2_scale(float scale) { return scale * 1.44269504088896341f; }

}  // namespace

hipError_t launch_kv_append(const AttnDims& s, const void* k_new, const void* v_new,
                            const int32_t* cu_q, const int32_t* kv_len, const int32_t* bt,
                            void* kc, void* vc, int max_q_per_seq, hipStream_t st) {
  const dim3 grid((unsigned)max_q_per_seq, (unsigned)s.B);
  if (s.d == 128)
    hipLaunchKernelGGL(kv_append_kernel<128>, grid, dim3(128), 0, st, (const uint16_t*)k_new,
                       (const uint16_t*)v_new, cu_q, kv_len, bt, (uint16_t*)kc, (uint16_t*)vc,
                       s.nkv, s.max_pages);
  else
    hipLaunchKernelGGL(kv_append_kernel<64>, grid, dim3(128), 0, st, (const uint16_t*)k_new,
                       (const uint16_t*)v_new, cu_q, kv_len, bt, (uint16_t*)kc, (uint16_t*)vc,
                       s.nkv, s.max_pages);
  return hipGetLastError();
}

hipError_t launch_attn_prefill(const AttnDims& s, const void* q, const int32_t* cu_q,
                               const int32_t* kv_len, const int32_t* bt, const void* kc,
                               const void* vc, void* out, float* lse, int max_q_per_seq,
                               hipStream_t st) {
  const int ppw = 16 / (s.nq / s.nkv);
  const int per_wg = 4 * ppw;
  const dim3 grid((unsigned)((max_q_per_seq + per_wg - 1) / per_wg), (unsigned)s.nkv,
                  (unsigned)s.B);
  const float c2 = base2_scale(s.scale);
  if (s.d == 128)
    hipLaunchKernelGGL(bi_attn_prefill_kernel<128>, grid, dim3(256), 0, st, (const uint16_t*)q,
                       cu_q, kv_len, bt, (const uint16_t*)kc, (const uint16_t*)vc,
                       (uint16_t*)out, lse, s.nq, s.nkv, s.max_pages, c2);
  else
    hipLaunchKernelGGL(bi_attn_prefill_kernel<64>, grid, dim3(256), 0, st, (const uint16_t*)q,
                       cu_q, kv_len, bt, (const uint16_t*)kc, (const uint16_t*)vc,
                       (uint16_t*)out, lse, s.nq, s.nkv, s.max_pages, c2);
  return hipGetLastError();
}

hipError_t launch_attn_decode(const AttnDims& s, const void* q, const int32_t* kv_len,
                              const int32_t* bt, const void* kc, const void* vc, void* out,
                              float* lse, int max_splits, float* ws, hipStream_t st) {
  const int64_t units = (int64_t)s.B * s.nkv * max_splits;
  const dim3 grid1((unsigned)((units + 3) / 4)), grid2((unsigned)((int64_t)s.B * s.nq));
  const float c2 = base2_scale(s.scale);
  if (s.d == 128) {
    hipLaunchKernelGGL(bi_attn_decode_partial_kernel<128>, grid1, dim3(256), 0, st,
                       (const uint16_t*)q, kv_len, bt, (const uint16_t*)kc, (const uint16_t*)vc,
                       ws, s.B, s.nq, s.nkv, s.max_pages, max_splits, c2);
    hipLaunchKernelGGL(bi_attn_combine_kernel<128>, grid2, dim3(128), 0, st, (const float*)ws,
                       kv_len, (uint16_t*)out, lse, s.nq, max_splits, kSplit);
  } else {
    hipLaunchKernelGGL(bi_attn_decode_partial_kernel<64>, grid1, dim3(256), 0, st,
                       (const uint16_t*)q, kv_len, bt, (const uint16_t*)kc, (const uint16_t*)vc,
                       ws, s.B, s.nq, s.nkv, s.max_pages, max_splits, c2);
    hipLaunchKernelGGL(bi_attn_combine_kernel<64>, grid2, dim3(64), 0, st, (const float*)ws,
                       kv_len, (uint16_t*)out, lse, s.nq, max_splits, kSplit);
  }
  return hipGetLastError();
}

int attn_splitkv_auto(int B, int nkv, int max_kv_len) {
  // The usual decode heuristic: enough splits for about two waves per SIMD
  // over the whole GPU, never shorter than 32 keys.
  const int64_t pairs = (int64_t)B * nkv;
  int64_t n = (2048 + pairs - 1) / (pairs > 0 ? pairs : 1);
  const int64_t most = (max_kv_len + 31) / 32;
  if (n > most) n = most;
  if (n > 256) n = 256;
  if (n < 1) n = 1;
  return (int)n;
}

hipError_t launch_attn_decode_splitkv(const AttnDims& s, const void* q, const int32_t* kv_len,
                                      const int32_t* bt, const void* kc, const void* vc, void* out,
                                      float* lse, int max_kv_len, int num_splits, float* ws,
                                      hipStream_t st) {
  int split_len = (max_kv_len + num_splits - 1) / num_splits;
  split_len = (split_len + 31) / 32 * 32;
  const int nsplit = (max_kv_len + split_len - 1) / split_len;
  const int64_t units = (int64_t)s.B * s.nkv * nsplit;
  const dim3 grid1((unsigned)((units + 3) / 4)), grid2((unsigned)((int64_t)s.B * s.nq));
  const float c2 = base2_scale(s.scale);
  if (s.d == 128) {
    hipLaunchKernelGGL(bix_attn_decode_splitkv_kernel<128>, grid1, dim3(256), 0, st,
                       (const uint16_t*)q, kv_len, bt, (const uint16_t*)kc, (const uint16_t*)vc,
                       ws, s.B, s.nq, s.nkv, s.max_pages, nsplit, split_len, c2);
    hipLaunchKernelGGL(bi_attn_combine_kernel<128>, grid2, dim3(128), 0, st, (const float*)ws,
                       kv_len, (uint16_t*)out, lse, s.nq, nsplit, split_len);
  } else {
    hipLaunchKernelGGL(bix_attn_decode_splitkv_kernel<64>, grid1, dim3(256), 0, st,
                       (const uint16_t*)q, kv_len, bt, (const uint16_t*)kc, (const uint16_t*)vc,
                       ws, s.B, s.nq, s.nkv, s.max_pages, nsplit, split_len, c2);
    hipLaunchKernelGGL(bi_attn_combine_kernel<64>, grid2, dim3(64), 0, st, (const float*)ws,
                       kv_len, (uint16_t*)out, lse, s.nq, nsplit, split_len);
  }
  return hipGetLastError();
}

}  // namespace bi
