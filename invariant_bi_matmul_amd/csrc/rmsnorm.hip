// RMSNorm kernels.
//
// bi_rmsnorm_kernel follows the RMSNorm row of the approach table in
// "Defeating Nondeterminism in LLM Inference" (mobiles-han.blogspot.com
// summary): the reduction is always data-parallel -- one workgroup owns one
// whole row -- so a row's order of additions never depends on how many rows
// the call has.  The order is fixed by `hidden` alone:
//   1. thread t owns the 16-byte vectors t, t+256, t+512, ... of the row and
//      adds their squares sequentially in element order (fp32);
//   2. a wave64 xor-butterfly (offsets 32,16,...,1) -- every lane ends with the
//      same bits because IEEE addition commutes;
//   3. the four waves' sums are added in wave order through LDS.
// Then rstd = 1/sqrt(sum/hidden + eps) and y = bf16((x*rstd)*gamma).
//
// bix_rmsnorm_splitrow_* is the non-invariant comparator from the problem
// column of the same row: when there are few rows, each row's reduction is
// split over several workgroups, so the order depends on the row count.
#include "common.h"
#include "kernels.h"

namespace bi {
namespace {

constexpr int kRmsThreads = 256;

template <int VPT>
__global__ __launch_bounds__(kRmsThreads) void bi_rmsnorm_kernel(
    const u32x4* x, const u32x4* gamma, u32x4* y, float* rstd, int hidden, float eps) {
  const int nvec = hidden >> 3;
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const u32x4* xr = x + row * nvec;
  u32x4 v[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int idx = tid + i * kRmsThreads;
    v[i] = idx < nvec ? __builtin_nontemporal_load(xr + idx) : u32x4{0u, 0u, 0u, 0u};
  }
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = bf16_lo(v[i][j]);
      const float b = bf16_hi(v[i][j]);
      ss = ss + a * a;
      ss = ss + b * b;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss = ss + __shfl_xor(ss, off);
  __shared__ float part[kRmsThreads / kWave];
  if ((tid & (kWave - 1)) == 0) part[tid / kWave] = ss;
  __syncthreads();
  const float tot = ((part[0] + part[1]) + part[2]) + part[3];
  const float r = 1.0f / sqrtf(tot / (float)hidden + eps);
  if (rstd != nullptr && tid == 0) rstd[row] = r;
  u32x4* yr = y + row * nvec;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int idx = tid + i * kRmsThreads;
    if (idx < nvec) {
      const u32x4 g = gamma[idx];
      u32x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a = (bf16_lo(v[i][j]) * r) * bf16_lo(g[j]);
        const float b = (bf16_hi(v[i][j]) * r) * bf16_hi(g[j]);
        o[j] = pack_bf16x2(a, b);
      }
      __builtin_nontemporal_store(o, yr + idx);
    }
  }
}

// ---- comparator: split-row reduction --------------------------------------

// Partial sum of squares of chunk blockIdx.y of row blockIdx.x.
__global__ __launch_bounds__(kRmsThreads) void bix_rmsnorm_partial_kernel(const u32x4* x,
                                                                          int hidden, int chunks,
                                                                          float* ws) {
  const int nvec = hidden >> 3;
  const int64_t row = blockIdx.x;
  const int c = blockIdx.y;
  const int per = (nvec + chunks - 1) / chunks;
  const int lo = c * per;
  const int hi = min(nvec, lo + per);
  float ss = 0.0f;
  for (int idx = lo + (int)threadIdx.x; idx < hi; idx += kRmsThreads) {
    const u32x4 v = x[row * nvec + idx];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = bf16_lo(v[j]), b = bf16_hi(v[j]);
      ss = ss + a * a;
      ss = ss + b * b;
    }
  }
  // tree in the opposite direction to the invariant kernel (1,2,...,32)
#pragma unroll
  for (int off = 1; off <= 32; off <<= 1) ss = ss + __shfl_xor(ss, off);
  __shared__ float part[kRmsThreads / kWave];
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = ss;
  __syncthreads();
  if (threadIdx.x == 0) ws[row * 64 + c] = (part[0] + part[1]) + (part[2] + part[3]);
}

__global__ __launch_bounds__(kRmsThreads) void bix_rmsnorm_apply_kernel(
    const u32x4* x, const u32x4* gamma, u32x4* y, float* rstd, int hidden, float eps, int chunks,
    const float* ws) {
  const int nvec = hidden >> 3;
  const int64_t row = blockIdx.x;
  float tot = 0.0f;
  for (int c = 0; c < chunks; ++c) tot = tot + ws[row * 64 + c];
  const float r = 1.0f / sqrtf(tot / (float)hidden + eps);
  if (rstd != nullptr && threadIdx.x == 0) rstd[row] = r;
  for (int idx = threadIdx.x; idx < nvec; idx += kRmsThreads) {
    const u32x4 v = x[row * nvec + idx];
    const u32x4 g = gamma[idx];
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o[j] = pack_bf16x2((bf16_lo(v[j]) * r) * bf16_lo(g[j]), (bf16_hi(v[j]) * r) * bf16_hi(g[j]));
    }
    y[row * nvec + idx] = o;
  }
}

}  // namespace

hipError_t launch_rmsnorm(const void* x, const void* gamma, void* y, float* rstd, int64_t rows,
                          int hidden, float eps, hipStream_t st) {
  const int nvec = hidden / 8;
  const int vpt = (nvec + kRmsThreads - 1) / kRmsThreads;  // a function of hidden only
  const dim3 grid((unsigned)rows), block(kRmsThreads);
  const u32x4* xv = (const u32x4*)x;
  const u32x4* gv = (const u32x4*)gamma;
  u32x4* yv = (u32x4*)y;
  if (vpt <= 1)
    hipLaunchKernelGGL(bi_rmsnorm_kernel<1>, grid, block, 0, st, xv, gv, yv, rstd, hidden, eps);
  else if (vpt == 2)
    hipLaunchKernelGGL(bi_rmsnorm_kernel<2>, grid, block, 0, st, xv, gv, yv, rstd, hidden, eps);
  else if (vpt <= 4)
    hipLaunchKernelGGL(bi_rmsnorm_kernel<4>, grid, block, 0, st, xv, gv, yv, rstd, hidden, eps);
  else
    hipLaunchKernelGGL(bi_rmsnorm_kernel<8>, grid, block, 0, st, xv, gv, yv, rstd, hidden, eps);
  return hipGetLastError();
}

int rmsnorm_splitrow_auto_chunks(int64_t rows) {
  // Few rows leave most CUs idle, so split each row: about 1024 workgroups.
  int64_t c = rows > 0 ? (1024 + rows - 1) / rows : 1;
  if (c < 1) c = 1;
  if (c > 16) c = 16;
  return (int)c;
}

hipError_t launch_rmsnorm_splitrow(const void* x, const void* gamma, void* y, float* rstd,
                                   int64_t rows, int hidden, float eps, int chunks, float* ws,
                                   hipStream_t st) {
  hipLaunchKernelGGL(bix_rmsnorm_partial_kernel, dim3((unsigned)rows, (unsigned)chunks),
                     dim3(kRmsThreads), 0, st, (const u32x4*)x, hidden, chunks, ws);
  hipLaunchKernelGGL(bix_rmsnorm_apply_kernel, dim3((unsigned)rows), dim3(kRmsThreads), 0, st,
                     (const u32x4*)x, (const u32x4*)gamma, (u32x4*)y, rstd, hidden, eps, chunks,
                     (const float*)ws);
  return hipGetLastError();
}

}  // namespace bi
