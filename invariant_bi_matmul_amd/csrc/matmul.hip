// Dense bf16 matmul, C[m,n] = sum_k A[m,k] W[k,n], fp32 accumulation.
//
// bi_matmul_kernel follows the MatMul row of the approach table in "Defeating
// Nondeterminism in LLM Inference" (mobiles-han.blogspot.com summary): one
// kernel configuration, compiled ahead, is used for every shape and batch
// size.  Here that is one tile (BM x BN x BK = 256 x 256 x 64, eight wave64s
// of 128 x 64 each), one MFMA instruction (v_mfma_f32_32x32x16_bf16), one
// k order (k-tiles ascending, 16-wide MFMA steps ascending inside a tile) and
// no split-K.  M only decides how many tiles exist; rows past M are computed
// from a clamped (valid) row and never stored, and MFMA rows do not interact,
// so a row's bits are the same for every M and every position in a tile.
//
// Data path per k-tile: global -> registers -> LDS (double buffered) -> MFMA.
// A [M,K] is k-contiguous and goes to LDS as is.  W [K,N] is n-contiguous;
// each thread loads an 8(k) x 4(n) block and transposes it in registers so
// that W is stored in LDS k-contiguous per column, which is the operand layout
// MFMA wants.  16-byte LDS chunks are XOR-swizzled by row to spread banks.
//
// bix_matmul_* is the non-invariant comparator from the problem column of the
// same row: split-K with a split count chosen from the grid size (so from M),
// fp32 partials summed by a second kernel.
#include "common.h"
#include "kernels.h"

namespace bi {
namespace {

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct MMTile {
  static constexpr int BM = BM_, BN = BN_, BK = kMatmulBK;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int NT = kWave * WAVES_M * WAVES_N;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int MI = WM / 32, NI = WN / 32;
  static constexpr int A_LOADS = BM * (BK / 8) / NT;          // 16-byte chunks per thread
  static constexpr int W_BLOCKS = (BK / 8) * (BN / 4) / NT;   // 8x4 blocks per thread
  static constexpr int LDS_A = BM * BK * 2;                   // bytes per stage
  static constexpr int LDS_B = BN * BK * 2;
  static constexpr int LDS_STAGE = LDS_A + LDS_B;
  static_assert(A_LOADS * NT == BM * (BK / 8), "A tile must split evenly over threads");
  static_assert(W_BLOCKS * NT == (BK / 8) * (BN / 4), "W tile must split evenly over threads");
  static_assert(MI * 32 == WM && NI * 32 == WN, "wave tile must be a multiple of 32");
};

// The one configuration.
using Tile = MMTile<256, 256, 2, 4>;

// 16-byte chunk swizzle within a 128-byte LDS row (BK = 64 bf16).
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

template <class T, bool SPLIT>
__global__ __launch_bounds__(T::NT) void bi_matmul_kernel(const uint16_t* __restrict__ A,
                                                          const uint16_t* __restrict__ W,
                                                          void* __restrict__ C, int M, int N,
                                                          int K, int out_f32, int kt_per_split) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * T::LDS_STAGE];

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

  u32x4 ra[T::A_LOADS];
  u32x2 rw[T::W_BLOCKS][8];

  auto gload = [&](int kt) {
    const int kb0 = kt * T::BK;
#pragma unroll
    for (int i = 0; i < T::A_LOADS; ++i) {
      const int c = tid + i * T::NT;
      const int row = c >> 3, ch = c & 7;
      const int gr = min(m0 + row, M - 1);
      ra[i] = *(const u32x4*)(A + (int64_t)gr * K + kb0 + ch * 8);
    }
#pragma unroll
    for (int b = 0; b < T::W_BLOCKS; ++b) {
      const int blk = tid + b * T::NT;
      const int nb = blk % (T::BN / 4), kb = blk / (T::BN / 4);
      const int gn = min(n0 + nb * 4, N - 4);
      const uint16_t* src = W + (int64_t)(kb0 + kb * 8) * N + gn;
#pragma unroll
      for (int r = 0; r < 8; ++r) rw[b][r] = *(const u32x2*)(src + (int64_t)r * N);
    }
  };

  auto sstore = [&](int stage) {
    uint8_t* As = smem + stage * T::LDS_STAGE;
    uint8_t* Bs = As + T::LDS_A;
#pragma unroll
    for (int i = 0; i < T::A_LOADS; ++i) {
      const int c = tid + i * T::NT;
      const int row = c >> 3, ch = c & 7;
      *(u32x4*)(As + row * 128 + ((ch ^ swz(row)) << 4)) = ra[i];
    }
#pragma unroll
    for (int b = 0; b < T::W_BLOCKS; ++b) {
      const int blk = tid + b * T::NT;
      const int nb = blk % (T::BN / 4), kb = blk / (T::BN / 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int hw = j >> 1;
        u32x4 t;
        if (j & 1) {
          t = u32x4{pack_hi(rw[b][0][hw], rw[b][1][hw]), pack_hi(rw[b][2][hw], rw[b][3][hw]),
                    pack_hi(rw[b][4][hw], rw[b][5][hw]), pack_hi(rw[b][6][hw], rw[b][7][hw])};
        } else {
          t = u32x4{pack_lo(rw[b][0][hw], rw[b][1][hw]), pack_lo(rw[b][2][hw], rw[b][3][hw]),
                    pack_lo(rw[b][4][hw], rw[b][5][hw]), pack_lo(rw[b][6][hw], rw[b][7][hw])};
        }
        const int n = nb * 4 + j;
        *(u32x4*)(Bs + n * 128 + ((kb ^ swz(n)) << 4)) = t;
      }
    }
  };

  f32x16 acc[T::MI][T::NI];
#pragma unroll
  for (int mi = 0; mi < T::MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < T::NI; ++ni) acc[mi][ni] = f32x16{};

  auto compute = [&](int stage) {
    const uint8_t* As = smem + stage * T::LDS_STAGE;
    const uint8_t* Bs = As + T::LDS_A;
#pragma unroll
    for (int kk = 0; kk < T::BK / 16; ++kk) {
      const int ch = 2 * kk + (lane >> 5);
      bf16x8 af[T::MI], bw[T::NI];
#pragma unroll
      for (int mi = 0; mi < T::MI; ++mi) {
        const int r = wave_m * T::WM + mi * 32 + (lane & 31);
        af[mi] = as_bf16x8(*(const u32x4*)(As + r * 128 + ((ch ^ swz(r)) << 4)));
      }
#pragma unroll
      for (int ni = 0; ni < T::NI; ++ni) {
        const int n = wave_n * T::WN + ni * 32 + (lane & 31);
        bw[ni] = as_bf16x8(*(const u32x4*)(Bs + n * 128 + ((ch ^ swz(n)) << 4)));
      }
#pragma unroll
      for (int mi = 0; mi < T::MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < T::NI; ++ni) acc[mi][ni] = mfma32(af[mi], bw[ni], acc[mi][ni]);
    }
  };

  if (kt0 < kt1) {
    gload(kt0);
    sstore(0);
    __syncthreads();
    for (int kt = kt0; kt < kt1; ++kt) {
      const int s = (kt - kt0) & 1;
      const bool more = kt + 1 < kt1;
      if (more) gload(kt + 1);
      compute(s);
      if (more) sstore(s ^ 1);
      __syncthreads();
    }
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
