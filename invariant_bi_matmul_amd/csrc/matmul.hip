// Dense bf16 matmul, C[m,n] = sum_k A[m,k] W[k,n], fp32 accumulation.
//
// bi_matmul_kernel follows the MatMul row of the approach table in "Defeating
// Nondeterminism in LLM Inference" (mobiles-han.blogspot.com summary): one
// kernel configuration, compiled ahead, is used for every shape and batch
// size.  Here that is one tile (BM x BN x BK = 256 x 128 x 64, eight wave64s of
// 64 x 64 each), one MFMA instruction (v_mfma_f32_32x32x16_bf16), one k order
// (k-tiles ascending, 16-wide MFMA steps ascending inside a tile) and no
// split-K.  M only decides how many tiles exist; rows past M are computed from
// a clamped (valid) row and never stored, and MFMA rows do not interact, so a
// row's bits are the same for every M and every position in a tile.
//
// Data path per k-tile: global -> LDS by direct loads (global_load_lds, 16
// bytes per lane, no register staging) into a ring of LDS stages -> MFMA
// operands.  A [M,K] is stored k-contiguous with a row-dependent XOR swizzle of
// its 16-byte chunks.  W [K,N] stays in its natural n-contiguous layout and
// the B operand, which needs 8 consecutive k per lane, is read with the
// transposing LDS load ds_read_b64_tr_b16 (lane 4a+c of each 16-lane group
// receives column c of the rows its group-mates a, a+4, a+8, a+12 address).
// The LDS ring has three stages (144 KiB), so loads run two k-tiles ahead,
// enough to cover the latency of reads that miss the caches.
//
// bix_matmul_* is the non-invariant comparator from the problem column of the
// same row: split-K with a split count chosen from the grid size (so from M),
// fp32 partials summed by a second kernel.
#include "common.h"
#include "kernels.h"

namespace bi {
namespace {

template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int STAGES_, bool PREFETCH_ = true>
struct MMTile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_;
  static constexpr bool PREFETCH = PREFETCH_;  // read step kk+1's fragments during step kk
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int NT = kWave * WAVES_M * WAVES_N;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int MI = WM / 32, NI = WN / 32;
  static constexpr int A_BYTES = BM * BK * 2;        // per stage
  static constexpr int W_BYTES = BK * BN * 2;
  static constexpr int STAGE_BYTES = A_BYTES + W_BYTES;
  static constexpr int A_LOADS = A_BYTES / 16 / NT;  // 16-byte direct loads per thread
  static constexpr int W_LOADS = W_BYTES / 16 / NT;
  static constexpr int LOADS = A_LOADS + W_LOADS;
  static constexpr int W_ROW = BN * 2;               // bytes per k row of W in LDS
  static constexpr int A_ROW = BK * 2;               // bytes per row of A in LDS
  static constexpr int A_CPR = BK / 8;               // 16-byte chunks per A row
  static_assert(BK == 32 || BK == 64 || BK == 128, "BK");
  static_assert(A_LOADS * NT * 16 == A_BYTES && W_LOADS * NT * 16 == W_BYTES, "tile/threads");
  static_assert(MI * 32 == WM && NI * 32 == WN, "wave tile must be a multiple of 32");
  static_assert(BN % 64 == 0, "W rows must hold whole 128-byte swizzle groups");
  static_assert(STAGES >= 2 && STAGES * STAGE_BYTES <= 160 * 1024, "LDS");
  static_assert((STAGES - 2) * LOADS <= 63, "vmcnt range");
};

// The one configuration.
using Tile = MMTile<256, 128, 64, 4, 2, 3, true>;

// A in LDS: [BM rows][BK/8 chunks of 16 B]; chunk c of row r sits at
// c ^ swz_a(r), chosen so that the 8 rows an MFMA operand read touches per
// 128-byte bank window fall on 8 different 16-byte bank groups.
template <int BK>
__device__ __forceinline__ int swz_a(int r) {
  if constexpr (BK == 32) return (r >> 1) & 3;
  else if constexpr (BK == 64) return (r ^ (r >> 3)) & 7;
  else return r & 7;
}
// W in LDS: [BK rows][BN/8 chunks]; chunk c of k row k sits at c ^ swz_w(k), so
// that the four k rows read by one transposed load land in distinct banks.
__device__ __forceinline__ int swz_w(int k) { return (k & 3) << 1; }

template <class T, bool SPLIT>
__global__ __launch_bounds__(T::NT) void bi_matmul_kernel(const uint16_t* __restrict__ A,
                                                          const uint16_t* __restrict__ W,
                                                          void* __restrict__ C, int M, int N,
                                                          int K, int out_f32, int kt_per_split) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[T::STAGES * T::STAGE_BYTES];

  const int tiles_m = (M + T::BM - 1) / T::BM;
  const int tiles_n = (N + T::BN - 1) / T::BN;
  const uint32_t id = xcd_contiguous_id(blockIdx.x, (uint32_t)(tiles_m * tiles_n));
  const int tm = (int)(id % (uint32_t)tiles_m);  // consecutive ids walk down M first
  const int tn = (int)(id / (uint32_t)tiles_m);
  const int m0 = tm * T::BM, n0 = tn * T::BN;

  int kt0 = 0, kt1 = K / T::BK;
  if (SPLIT) {
    kt0 = (int)blockIdx.z * kt_per_split;
    kt1 = min(kt1, kt0 + kt_per_split);
  }

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wave_m = wave / T::WAVES_N, wave_n = wave % T::WAVES_N;

  // Per-thread global sources of its direct loads (k offset added per tile).
  // Load i of wave w fills the 1 KiB LDS block (i*NT + w*64)*16 of the stage;
  // lane l of it lands at chunk q = i*NT + w*64 + l.
  const uint16_t* a_src[T::A_LOADS];
#pragma unroll
  for (int i = 0; i < T::A_LOADS; ++i) {
    const int q = i * T::NT + wave * kWave + lane;
    const int row = q / T::A_CPR, c = (q % T::A_CPR) ^ swz_a<T::BK>(q / T::A_CPR);
    a_src[i] = A + (int64_t)min(m0 + row, M - 1) * K + c * 8;
  }
  const uint16_t* w_src[T::W_LOADS];
#pragma unroll
  for (int i = 0; i < T::W_LOADS; ++i) {
    const int q = i * T::NT + wave * kWave + lane;
    const int k = q / (T::BN / 8), c = (q % (T::BN / 8)) ^ swz_w(q / (T::BN / 8));
    w_src[i] = W + (int64_t)k * N + min(n0 + c * 8, N - 8);
  }

  auto issue = [&](int kt, int stage) {
    const uint32_t base = (uint32_t)(uintptr_t)(smem + stage * T::STAGE_BYTES);
    const int64_t ka = (int64_t)kt * T::BK;
#pragma unroll
    for (int i = 0; i < T::A_LOADS; ++i)
      lds_dma16(a_src[i] + ka, base + (i * T::NT + wave * kWave) * 16);
    const int64_t kw = ka * N;
#pragma unroll
    for (int i = 0; i < T::W_LOADS; ++i)
      lds_dma16(w_src[i] + kw, base + T::A_BYTES + (i * T::NT + wave * kWave) * 16);
  };

  f32x16 acc[T::MI][T::NI];
#pragma unroll
  for (int mi = 0; mi < T::MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < T::NI; ++ni) acc[mi][ni] = f32x16{};

  // Operand fragments of one 16-wide k step, read from one LDS stage.
  const int g16 = lane >> 4, i16 = lane & 15;
  auto frags = [&](const uint8_t* As, const uint8_t* Ws, int kk, bf16x8 (&af)[T::MI],
                   bf16x8 (&bw)[T::NI]) {
    const int ch = 2 * kk + (lane >> 5);
#pragma unroll
    for (int mi = 0; mi < T::MI; ++mi) {
      const int r = wave_m * T::WM + mi * 32 + (lane & 31);
      af[mi] = as_bf16x8(*(const u32x4*)(As + r * T::A_ROW + ((ch ^ swz_a<T::BK>(r)) << 4)));
    }
#pragma unroll
    for (int ni = 0; ni < T::NI; ++ni) {
      // B operand: lane l needs W[16kk + 8(l/32) + e][col + (l & 31)], e = 0..7.
      // Two transposed reads of 4 k rows each: within a 16-lane group, lane i
      // addresses k row base + i/4, columns 4(i%4)..+3 of the group's 16.
      const int nb = wave_n * T::WN + ni * 32 + 16 * (g16 & 1) + 4 * (i16 & 3);
      s16x4 v[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = 16 * kk + 8 * (g16 >> 1) + 4 * h + (i16 >> 2);
        const uint8_t* p = Ws + k * T::W_ROW + (((nb >> 3) ^ swz_w(k)) << 4) + (nb & 7) * 2;
        v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
      }
      const u32x4 u = u32x4{(uint32_t)(uint16_t)v[0][0] | ((uint32_t)(uint16_t)v[0][1] << 16),
                            (uint32_t)(uint16_t)v[0][2] | ((uint32_t)(uint16_t)v[0][3] << 16),
                            (uint32_t)(uint16_t)v[1][0] | ((uint32_t)(uint16_t)v[1][1] << 16),
                            (uint32_t)(uint16_t)v[1][2] | ((uint32_t)(uint16_t)v[1][3] << 16)};
      bw[ni] = as_bf16x8(u);
    }
  };
  // k steps in ascending order.  With PREFETCH the fragments of step kk+1 are
  // read while the MFMAs of step kk run: each step is its own scheduling
  // region in which LDS reads and MFMAs alternate one for one.
  auto compute = [&](int stage) {
    const uint8_t* As = smem + stage * T::STAGE_BYTES;
    const uint8_t* Ws = As + T::A_BYTES;
    bf16x8 af[2][T::MI], bw[2][T::NI];
    if (T::PREFETCH) frags(As, Ws, 0, af[0], bw[0]);
#pragma unroll
    for (int kk = 0; kk < T::BK / 16; ++kk) {
      if (T::PREFETCH) __builtin_amdgcn_sched_barrier(0);
      if (!T::PREFETCH) frags(As, Ws, kk, af[kk & 1], bw[kk & 1]);
      else if (kk + 1 < T::BK / 16) frags(As, Ws, kk + 1, af[(kk + 1) & 1], bw[(kk + 1) & 1]);
#pragma unroll
      for (int mi = 0; mi < T::MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < T::NI; ++ni)
          acc[mi][ni] = mfma32(af[kk & 1][mi], bw[kk & 1][ni], acc[mi][ni]);
      if (T::PREFETCH) {
        if (kk + 1 < T::BK / 16) {
#pragma unroll
          for (int i = 0; i < T::MI * T::NI; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // STAGES-deep ring filled by direct global->LDS loads.  Every iteration
  // issues exactly one tile (the index is clamped at the end, re-loading the
  // last tile into a stage nobody reads again), so the vector-memory counter
  // says exactly when tile k has landed: at most STAGES-2 younger tiles may be
  // outstanding.  One barrier per tile both publishes tile k and retires the
  // stage read in the previous iteration, which is the one refilled next.
  const int nk = kt1 - kt0;
  if (nk > 0) {
#pragma unroll
    for (int s = 0; s < T::STAGES - 1; ++s) issue(kt0 + min(s, nk - 1), s);
    for (int k = 0; k < nk; ++k) {
      wait_vmcnt_le<(T::STAGES - 2) * T::LOADS>();
      __syncthreads();
      issue(kt0 + min(k + T::STAGES - 1, nk - 1), (k + T::STAGES - 1) % T::STAGES);
      compute(k % T::STAGES);
    }
    wait_vmcnt_le<0>();  // no LDS write may outlive the workgroup
  }

  // Epilogue: lane holds column (lane & 31) and rows 8*(r/4) + 4*(lane/32) + r%4.
#pragma unroll
  for (int mi = 0; mi < T::MI; ++mi) {
#pragma unroll
    for (int ni = 0; ni < T::NI; ++ni) {
      const int col = n0 + wave_n * T::WN + ni * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wave_m * T::WM + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < M && col < N) {
          const int64_t o = (int64_t)row * N + col;
          const float v = acc[mi][ni][r];
          if (SPLIT) {
            ((float*)C)[(int64_t)blockIdx.z * M * N + o] = v;
          } else if (out_f32) {
            ((float*)C)[o] = v;
          } else {
            ((uint16_t*)C)[o] = (uint16_t)f32_to_bf16(v);
          }
        }
      }
    }
  }
}

// Sum split-K partials in slice order, then round.
__global__ __launch_bounds__(256) void bix_matmul_reduce_kernel(const float* __restrict__ ws,
                                                                 void* __restrict__ C,
                                                                 int64_t count, int splits,
                                                                 int out_f32) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  float s = ws[i];
  for (int p = 1; p < splits; ++p) s = s + ws[(int64_t)p * count + i];
  if (out_f32)
    ((float*)C)[i] = s;
  else
    ((uint16_t*)C)[i] = (uint16_t)f32_to_bf16(s);
}

}  // namespace

hipError_t launch_matmul(const void* a, const void* w, void* c, bool c_f32, int64_t m, int64_t n,
                         int64_t k, hipStream_t st) {
  const int64_t tiles = ((m + Tile::BM - 1) / Tile::BM) * ((n + Tile::BN - 1) / Tile::BN);
  hipLaunchKernelGGL((bi_matmul_kernel<Tile, false>), dim3((unsigned)tiles), dim3(Tile::NT), 0, st,
                     (const uint16_t*)a, (const uint16_t*)w, c, (int)m, (int)n, (int)k,
                     c_f32 ? 1 : 0, 0);
  return hipGetLastError();
}

int matmul_splitk_auto(int64_t m, int64_t n, int64_t k) {
  // Enough slices to give every CU a workgroup, the usual small-M heuristic.
  const int64_t tiles = ((m + Tile::BM - 1) / Tile::BM) * ((n + Tile::BN - 1) / Tile::BN);
  int64_t s = (256 + tiles - 1) / (tiles > 0 ? tiles : 1);
  const int64_t kt = k / Tile::BK;
  if (s > 16) s = 16;
  if (s > kt) s = kt;
  if (s < 1) s = 1;
  return (int)s;
}

hipError_t launch_matmul_splitk(const void* a, const void* w, void* c, bool c_f32, int64_t m,
                                int64_t n, int64_t k, int split_k, float* ws, hipStream_t st) {
  const int64_t tiles = ((m + Tile::BM - 1) / Tile::BM) * ((n + Tile::BN - 1) / Tile::BN);
  const int kt = (int)(k / Tile::BK);
  const int per = (kt + split_k - 1) / split_k;
  const int used = (kt + per - 1) / per;  // slices that own at least one k-tile
  hipLaunchKernelGGL((bi_matmul_kernel<Tile, true>), dim3((unsigned)tiles, 1, (unsigned)used),
                     dim3(Tile::NT), 0, st, (const uint16_t*)a, (const uint16_t*)w, (void*)ws,
                     (int)m, (int)n, (int)k, 1, per);
  const int64_t count = m * n;
  hipLaunchKernelGGL(bix_matmul_reduce_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0,
                     st, (const float*)ws, c, count, used, c_f32 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace bi
