// Measurement kernels: nothing on the batch-invariant path calls them.
//
// bix_mfma_loop_kernel gives the MFMA ceiling at the clock the chip actually
// holds under matrix load: each wave runs rounds of four independent
// v_mfma_f32_32x32x16_bf16 chains on register operands, with no memory
// traffic, so the only limit is the matrix pipe and its clock.  Four chains
// of one 32-cycle MFMA each keep a chain's next MFMA 128 cycles behind its
// previous one, past the instruction's latency.
//
// bix_read_stream_kernel gives the HBM read ceiling: a grid-stride sweep of
// 16-byte loads, four in flight per lane, folded into one value that is
// stored only if it is a pattern the sweep never produces.
#include "common.h"
#include "kernels.h"

namespace bi {
namespace {

__global__ __launch_bounds__(256) void bix_mfma_loop_kernel(int64_t iters, float* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(0.001f * (float)(lane + j));
    b[j] = (__bf16)(0.002f * (float)(lane - j));
  }
  f32x16 acc[4] = {};
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = mfma32(a, b, acc[c]);
  }
  // Fold the accumulators and store only on a value they never take, so the
  // loop is kept but nothing is written.
  float t = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) t = t + acc[c][r];
  if (t == 12345.0f) sink[0] = t;
}

__global__ __launch_bounds__(256) void bix_read_stream_kernel(const u32x4* __restrict__ p,
                                                              int64_t n16, uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= p[i];
  const uint32_t t = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (t == 0x9E3779B9u && acc[0] == 0x7F4A7C15u) sink[0] = t;
}

}  // namespace

hipError_t launch_read_stream(const void* p, int64_t bytes, int workgroups, uint32_t* sink,
                              hipStream_t st) {
  hipLaunchKernelGGL(bix_read_stream_kernel, dim3((unsigned)workgroups), dim3(256), 0, st,
                     (const u32x4*)p, bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_mfma_loop(int64_t iters, int workgroups, float* sink, hipStream_t st) {
  hipLaunchKernelGGL(bix_mfma_loop_kernel, dim3((unsigned)workgroups), dim3(256), 0, st, iters,
                     sink);
  return hipGetLastError();
}

}  // namespace bi
