// Element-wise and per-row operations of a Llama-style decoder stack around
// the three batch-invariant kernels: token embedding gather, rotary position
// embedding, SwiGLU, residual add and greedy argmax; and the operand packing
// of the error-compensated matmul (fp32 -> bf16 hi/lo planes).
//
// None of them reduces across rows: every output element depends only on its
// own row's inputs (and, for the rotary embedding, on its position), through
// one fixed sequence of fp32 operations.  So each is batch-invariant by
// construction; the stack built from them and from RMSNorm, matmul and split-KV
// attention gives a sequence the same tokens and logits alone or in any batch.
//
// Numerics: built with -ffp-contract=off and no fast-math (one rounding per
// operation as written); bf16 results are rounded to nearest even by
// pack_bf16x2.  The transcendental functions are the HIP device library's
// sinf/cosf/powf/expf, called the same way for every element.
#include <stdint.h>

#include "common.h"
#include "kernels.h"

namespace bi {
namespace {

constexpr int kElemThreads = 256;

// out[t, :] = table[ids[t], :]; ids are clamped into [0, vocab).
__global__ __launch_bounds__(kElemThreads) void embed_kernel(const int32_t* __restrict__ ids,
                                                             const u32x4* __restrict__ table,
                                                             u32x4* __restrict__ out,
                                                             int64_t vocab, int chunks) {
  const int64_t t = blockIdx.x;
  int64_t id = ids[t];
  id = id < 0 ? 0 : (id >= vocab ? vocab - 1 : id);
  const u32x4* src = table + id * chunks;
  u32x4* dst = out + t * chunks;
  for (int c = threadIdx.x; c < chunks; c += kElemThreads) dst[c] = src[c];
}

// Rotary embedding, "rotate half" pairing: for head h of token t at position
// p and i < d/2, with a = x[i], b = x[i + d/2] and angle = p * theta^(-2i/d):
//   x[i] = a cos - b sin,  x[i + d/2] = a sin + b cos.
// Grid (tokens, n_q + n_kv); thread i owns pair i.  In place.
// Pair i of one head row: src[i], src[i + d/2] rotated by the angle of
// position p, written to dst (which may be src).
__device__ __forceinline__ void rope_pair(const uint16_t* src, uint16_t* dst, int i, int d, int p,
                                          float theta) {
  const int half = d / 2;
  const float inv_freq = powf(theta, -(float)(2 * i) / (float)d);
  const float angle = (float)p * inv_freq;
  const float s = sinf(angle), c = cosf(angle);
  const float a = bf16_to_f32(src[i]), b = bf16_to_f32(src[i + half]);
  const float ya = a * c - b * s;
  const float yb = a * s + b * c;
  dst[i] = (uint16_t)f32_to_bf16(ya);
  dst[i + half] = (uint16_t)f32_to_bf16(yb);
}

__global__ void rope_kernel(uint16_t* __restrict__ q, uint16_t* __restrict__ k,
                            const int32_t* __restrict__ pos, int nq, int nkv, int d,
                            float theta) {
  const int64_t t = blockIdx.x;
  const int h = blockIdx.y;
  const int i = threadIdx.x;
  if (i >= d / 2) return;
  uint16_t* x = h < nq ? q + (t * nq + h) * d : k + (t * nkv + (h - nq)) * d;
  rope_pair(x, x, i, d, pos[t], theta);
}

// The output row of a fused q|k|v projection ([nq + 2 nkv] heads of d) split
// into contiguous q, k and v, with the rotary embedding of rope_kernel applied
// to the q and k heads on the way (the same arithmetic).
__global__ void qkv_rope_kernel(const uint16_t* __restrict__ qkv, const int32_t* __restrict__ pos,
                                uint16_t* __restrict__ q, uint16_t* __restrict__ k,
                                uint16_t* __restrict__ v, int nq, int nkv, int d, float theta) {
  const int64_t t = blockIdx.x;
  const int h = blockIdx.y;
  const int i = threadIdx.x;
  if (i >= d / 2) return;
  const uint16_t* src = qkv + (t * (nq + 2 * nkv) + h) * d;
  if (h < nq + nkv) {
    uint16_t* dst = h < nq ? q + (t * nq + h) * d : k + (t * nkv + (h - nq)) * d;
    rope_pair(src, dst, i, d, pos[t], theta);
  } else {
    uint16_t* dst = v + (t * nkv + (h - nq - nkv)) * d;
    dst[i] = src[i];
    dst[i + d / 2] = src[i + d / 2];
  }
}

// out = bf16(silu(gate) * up), silu(g) = g / (1 + e^-g); eight elements per
// thread.
__device__ __forceinline__ u32x4 swiglu8(u32x4 g, u32x4 u) {
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float r[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float gv = h ? bf16_hi(g[j]) : bf16_lo(g[j]);
      const float uv = h ? bf16_hi(u[j]) : bf16_lo(u[j]);
      const float silu = gv / (1.0f + expf(-gv));
      r[h] = silu * uv;
    }
    o[j] = pack_bf16x2(r[0], r[1]);
  }
  return o;
}

__global__ __launch_bounds__(kElemThreads) void swiglu_kernel(const u32x4* __restrict__ gate,
                                                              const u32x4* __restrict__ up,
                                                              u32x4* __restrict__ out,
                                                              int64_t vecs) {
  for (int64_t v = (int64_t)blockIdx.x * kElemThreads + threadIdx.x; v < vecs;
       v += (int64_t)gridDim.x * kElemThreads)
    out[v] = swiglu8(gate[v], up[v]);
}

// The same over the output of a fused gate|up projection: row r of gu holds
// gate (f values) then up (f values); out is [rows, f].  fv = f / 8.
__global__ __launch_bounds__(kElemThreads) void swiglu_pair_kernel(const u32x4* __restrict__ gu,
                                                                   u32x4* __restrict__ out,
                                                                   int64_t vecs, int64_t fv) {
  for (int64_t v = (int64_t)blockIdx.x * kElemThreads + threadIdx.x; v < vecs;
       v += (int64_t)gridDim.x * kElemThreads) {
    const int64_t r = v / fv, c = v - r * fv;
    out[v] = swiglu8(gu[r * 2 * fv + c], gu[r * 2 * fv + fv + c]);
  }
}

// out = bf16(a + b); eight elements per thread.  out may alias a or b.
__global__ __launch_bounds__(kElemThreads) void add_kernel(const u32x4* a, const u32x4* b,
                                                           u32x4* out, int64_t vecs) {
  for (int64_t v = (int64_t)blockIdx.x * kElemThreads + threadIdx.x; v < vecs;
       v += (int64_t)gridDim.x * kElemThreads) {
    const u32x4 x = a[v], y = b[v];
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = pack_bf16x2(bf16_lo(x[j]) + bf16_lo(y[j]), bf16_hi(x[j]) + bf16_hi(y[j]));
    out[v] = o;
  }
}

// Greedy argmax of one fp32 row per workgroup: the largest value, the lowest
// index among equal values; NaN is never chosen, and a row with no number in
// it gives 0.  (value desc, index asc) is a total order on the candidates, so
// the result does not depend on how the scan is split or reduced.
struct Best {
  float v;
  int i;
};
__device__ __forceinline__ Best better(Best x, Best y) {
  if (y.v > x.v || (y.v == x.v && y.i < x.i)) return y;
  return x;
}
__global__ __launch_bounds__(kElemThreads) void argmax_kernel(const float* __restrict__ x,
                                                              int32_t* __restrict__ out,
                                                              int64_t n) {
  const float* row = x + (int64_t)blockIdx.x * n;
  Best b{-INFINITY, INT32_MAX};
  for (int64_t j = threadIdx.x; j < n; j += kElemThreads) b = better(b, Best{row[j], (int)j});
#pragma unroll
  for (int s = 1; s < kWave; s <<= 1) {
    const Best o{__shfl_xor(b.v, s), __shfl_xor(b.i, s)};
    b = better(b, o);
  }
  __shared__ Best part[kElemThreads / kWave];
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) part[wave] = b;
  __syncthreads();
  if (threadIdx.x == 0) {
    Best r = part[0];
    for (int w = 1; w < kElemThreads / kWave; ++w) r = better(r, part[w]);
    out[blockIdx.x] = r.i == INT32_MAX ? 0 : r.i;
  }
}

// Error-compensated operands: x (fp32) -> hi = bf16(x), lo = bf16(x - hi)
// (x - hi is exact in fp32).  A non-finite hi has lo = 0.
__device__ __forceinline__ void ec_split(float x, uint32_t& hi, uint32_t& lo) {
  hi = f32_to_bf16(x);
  const float h = bf16_to_f32((uint16_t)hi);
  lo = isfinite(h) ? f32_to_bf16(x - h) : 0u;
}
// a3 [m, 3k] = [hi(a) | hi(a) | lo(a)] row by row; one thread per element of a.
__global__ __launch_bounds__(kElemThreads) void ec_pack_a_kernel(const float* __restrict__ a,
                                                                 uint16_t* __restrict__ a3,
                                                                 int64_t m, int64_t k) {
  const int64_t total = m * k;
  for (int64_t i = (int64_t)blockIdx.x * kElemThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kElemThreads) {
    const int64_t r = i / k, c = i - r * k;
    uint32_t hi, lo;
    ec_split(a[i], hi, lo);
    uint16_t* row = a3 + r * 3 * k;
    row[c] = (uint16_t)hi;
    row[k + c] = (uint16_t)hi;
    row[2 * k + c] = (uint16_t)lo;
  }
}
// a2 [m, 2k] = [a | a] row by row for a bf16 a (whose lo is 0); k % 8 == 0,
// one thread per 16-byte vector of a.
__global__ __launch_bounds__(kElemThreads) void ec_pack_a_bf16_kernel(const u32x4* __restrict__ a,
                                                                      u32x4* __restrict__ a2,
                                                                      int64_t m, int64_t kv) {
  const int64_t total = m * kv;
  for (int64_t i = (int64_t)blockIdx.x * kElemThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kElemThreads) {
    const int64_t r = i / kv, c = i - r * kv;
    const u32x4 x = a[i];
    a2[r * 2 * kv + c] = x;
    a2[r * 2 * kv + kv + c] = x;
  }
}
// w3 [3k, n] = [hi(w); lo(w); hi(w)] stacked along k.
__global__ __launch_bounds__(kElemThreads) void ec_pack_w_kernel(const float* __restrict__ w,
                                                                 uint16_t* __restrict__ w3,
                                                                 int64_t k, int64_t n) {
  const int64_t total = k * n;
  for (int64_t i = (int64_t)blockIdx.x * kElemThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kElemThreads) {
    uint32_t hi, lo;
    ec_split(w[i], hi, lo);
    w3[i] = (uint16_t)hi;
    w3[total + i] = (uint16_t)lo;
    w3[2 * total + i] = (uint16_t)hi;
  }
}

unsigned elem_grid(int64_t vecs) {
  int64_t g = (vecs + kElemThreads - 1) / kElemThreads;
  if (g > 65536) g = 65536;
  return (unsigned)(g < 1 ? 1 : g);
}

}  // namespace

hipError_t launch_embed(const int32_t* ids, const void* table, void* out, int64_t tokens,
                        int64_t hidden, int64_t vocab, hipStream_t st) {
  hipLaunchKernelGGL(embed_kernel, dim3((unsigned)tokens), dim3(kElemThreads), 0, st, ids,
                     (const u32x4*)table, (u32x4*)out, vocab, (int)(hidden / 8));
  return hipGetLastError();
}

hipError_t launch_rope(void* q, void* k, const int32_t* pos, int64_t tokens, int nq, int nkv,
                       int d, float theta, hipStream_t st) {
  const int threads = ((d / 2 + kWave - 1) / kWave) * kWave;
  hipLaunchKernelGGL(rope_kernel, dim3((unsigned)tokens, (unsigned)(nq + nkv)), dim3(threads), 0,
                     st, (uint16_t*)q, (uint16_t*)k, pos, nq, nkv, d, theta);
  return hipGetLastError();
}

hipError_t launch_qkv_rope(const void* qkv, const int32_t* pos, void* q, void* k, void* v,
                           int64_t tokens, int nq, int nkv, int d, float theta, hipStream_t st) {
  const int threads = ((d / 2 + kWave - 1) / kWave) * kWave;
  hipLaunchKernelGGL(qkv_rope_kernel, dim3((unsigned)tokens, (unsigned)(nq + 2 * nkv)),
                     dim3(threads), 0, st, (const uint16_t*)qkv, pos, (uint16_t*)q, (uint16_t*)k,
                     (uint16_t*)v, nq, nkv, d, theta);
  return hipGetLastError();
}

hipError_t launch_swiglu_pair(const void* gu, void* out, int64_t rows, int64_t f, hipStream_t st) {
  const int64_t vecs = rows * f / 8;
  hipLaunchKernelGGL(swiglu_pair_kernel, dim3(elem_grid(vecs)), dim3(kElemThreads), 0, st,
                     (const u32x4*)gu, (u32x4*)out, vecs, f / 8);
  return hipGetLastError();
}

hipError_t launch_swiglu(const void* gate, const void* up, void* out, int64_t n, hipStream_t st) {
  const int64_t vecs = n / 8;
  hipLaunchKernelGGL(swiglu_kernel, dim3(elem_grid(vecs)), dim3(kElemThreads), 0, st,
                     (const u32x4*)gate, (const u32x4*)up, (u32x4*)out, vecs);
  return hipGetLastError();
}

hipError_t launch_add(const void* a, const void* b, void* out, int64_t n, hipStream_t st) {
  const int64_t vecs = n / 8;
  hipLaunchKernelGGL(add_kernel, dim3(elem_grid(vecs)), dim3(kElemThreads), 0, st,
                     (const u32x4*)a, (const u32x4*)b, (u32x4*)out, vecs);
  return hipGetLastError();
}

hipError_t launch_ec_pack_a(const float* a, void* a3, int64_t m, int64_t k, hipStream_t st) {
  hipLaunchKernelGGL(ec_pack_a_kernel, dim3(elem_grid(m * k)), dim3(kElemThreads), 0, st, a,
                     (uint16_t*)a3, m, k);
  return hipGetLastError();
}

hipError_t launch_ec_pack_a_bf16(const void* a, void* a2, int64_t m, int64_t k, hipStream_t st) {
  hipLaunchKernelGGL(ec_pack_a_bf16_kernel, dim3(elem_grid(m * (k / 8))), dim3(kElemThreads), 0,
                     st, (const u32x4*)a, (u32x4*)a2, m, k / 8);
  return hipGetLastError();
}

hipError_t launch_ec_pack_w(const float* w, void* w3, int64_t k, int64_t n, hipStream_t st) {
  hipLaunchKernelGGL(ec_pack_w_kernel, dim3(elem_grid(k * n)), dim3(kElemThreads), 0, st, w,
                     (uint16_t*)w3, k, n);
  return hipGetLastError();
}

hipError_t launch_argmax(const float* x, int32_t* out, int64_t rows, int64_t n, hipStream_t st) {
  hipLaunchKernelGGL(argmax_kernel, dim3((unsigned)rows), dim3(kElemThreads), 0, st, x, out, n);
  return hipGetLastError();
}

}  // namespace bi
