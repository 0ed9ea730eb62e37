// Measurement kernels: nothing on the batch-invariant path calls them.
//
// bix_mfma_loop_kernel gives the MFMA ceiling at the clock the chip actually
// holds under matrix load: each wave runs rounds of four independent
// v_mfma_f32_32x32x16_bf16 chains on register operands, with no memory
// traffic, so the only limit is the matrix pipe and its clock.  Four chains
// of one 32-cycle MFMA each keep a chain's next MFMA 128 cycles behind its
// previous one, past the instruction's latency.  The pipe's power, and so the
// clock the chip can hold, depends on the operand bits: with VARIED the four
// chains cycle through four operand pairs of hashed bits (random sign and
// mantissa, magnitude in [1/16, 1)), so that each MFMA's inputs differ from
// the previous one's as they do in a matmul; otherwise every MFMA takes the
// same smooth, slowly varying pair.
//
// bix_read_stream_kernel gives the HBM read ceiling the way the decode kernel
// reads: each wave pulls 8 KiB chunks (chunks w, w + NW, ... of the buffer)
// through a private LDS ring of 8 chunk slots by direct global->LDS loads,
// seven chunks in flight, and touches one value of each landed chunk.
#include "common.h"
#include "kernels.h"

namespace bi {
namespace {

__device__ __forceinline__ uint32_t mix32(uint32_t h) {
  h ^= h >> 16;
  h *= 0x7feb352du;
  h ^= h >> 15;
  h *= 0x846ca68bu;
  h ^= h >> 16;
  return h;
}

template <bool VARIED>
__global__ __launch_bounds__(256) void bix_mfma_loop_kernel(int64_t iters, float* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (VARIED) {
        const uint32_t h = mix32((uint32_t)(lane * 64 + j * 4 + p) * 2654435761u + 1u);
        // sign, exponent 123..126, 7 mantissa bits
        const uint16_t ab = (uint16_t)(((h & 1u) << 15) | ((123u + ((h >> 1) & 3u)) << 7) |
                                       ((h >> 3) & 0x7fu));
        const uint16_t bb = (uint16_t)((((h >> 10) & 1u) << 15) |
                                       ((123u + ((h >> 11) & 3u)) << 7) | ((h >> 13) & 0x7fu));
        a[p][j] = __builtin_bit_cast(__bf16, ab);
        b[p][j] = __builtin_bit_cast(__bf16, bb);
      } else {
        a[p][j] = (__bf16)(0.001f * (float)(lane + j));
        b[p][j] = (__bf16)(0.002f * (float)(lane - j));
      }
    }
  f32x16 acc[4] = {};
  int64_t i = 0;
  for (; i + 4 <= iters; i += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = mfma32(a[(u + c) & 3], b[(u + c) & 3], acc[c]);
  }
  for (; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = mfma32(a[c], b[c], acc[c]);
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

constexpr int kStreamChunk = 8192, kStreamRing = 8, kStreamWaves = 2;

__global__ __launch_bounds__(64 * kStreamWaves) void bix_read_stream_kernel(const uint8_t* buf,
                                                                           int64_t nchunks,
                                                                           uint32_t* sink) {
  constexpr int LOADS = kStreamChunk / 1024;  // 1 KiB direct loads per chunk
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kStreamWaves][kStreamRing * kStreamChunk];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t NW = (int64_t)gridDim.x * kStreamWaves;
  const int64_t w = (int64_t)blockIdx.x * kStreamWaves + wave;
  const int64_t mine = w < nchunks ? (nchunks - w + NW - 1) / NW : 0;  // chunks of this wave
  const uint32_t base = (uint32_t)(uintptr_t)ring[wave];
  auto issue = [&](int64_t i) {  // the wave's i-th chunk into slot i mod RING
    const uint8_t* src = buf + (w + i * NW) * kStreamChunk;
#pragma unroll
    for (int n = 0; n < LOADS; ++n)
      lds_dma16_sv(src + n * 1024, (uint32_t)lane * 16,
                   base + (uint32_t)((i % kStreamRing) * kStreamChunk + n * 1024));
  };
  for (int64_t i = 0; i < kStreamRing - 1 && i < mine; ++i) issue(i);
  uint32_t acc = 0;
  for (int64_t i = 0; i < mine; ++i) {
    // chunk i has landed once at most the younger in-flight chunks remain
    if (i + kStreamRing - 1 <= mine) wait_vmcnt_le<(kStreamRing - 2) * LOADS>();
    else wait_vmcnt_le<0>();
    acc ^= *(const uint32_t*)(ring[wave] + (i % kStreamRing) * kStreamChunk + lane * 16);
    lds_reads_done();  // slot (i-1) mod RING is refilled next: its read is complete
    if (i + kStreamRing - 1 < mine) issue(i + kStreamRing - 1);
  }
  wait_vmcnt_le<0>();
  if (acc == 0x9E3779B9u && lane == 63) sink[0] = acc;
}

}  // namespace

hipError_t launch_read_stream(const void* p, int64_t bytes, int workgroups, uint32_t* sink,
                              hipStream_t st) {
  hipLaunchKernelGGL(bix_read_stream_kernel, dim3((unsigned)workgroups), dim3(64 * kStreamWaves),
                     0, st, (const uint8_t*)p, bytes / kStreamChunk, sink);
  return hipGetLastError();
}

hipError_t launch_mfma_loop(int64_t iters, int workgroups, bool varied, float* sink,
                            hipStream_t st) {
  if (varied)
    hipLaunchKernelGGL(bix_mfma_loop_kernel<true>, dim3((unsigned)workgroups), dim3(256), 0, st,
                       iters, sink);
  else
    hipLaunchKernelGGL(bix_mfma_loop_kernel<false>, dim3((unsigned)workgroups), dim3(256), 0, st,
                       iters, sink);
  return hipGetLastError();
}

}  // namespace bi
