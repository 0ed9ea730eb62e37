// Dense bf16 matmul, C[m,n] = sum_k A[m,k] W[k,n], fp32 accumulation.
//
// bi_matmul_kernel follows the MatMul row of the approach table in "Defeating
// Nondeterminism in LLM Inference" (mobiles-han.blogspot.com summary): one
// kernel configuration, compiled ahead, is used for every shape and batch
// size.  Here the configuration is what decides an element's bits: one MFMA
// instruction (v_mfma_f32_32x32x16_bf16), one k order (64-wide k-tiles
// ascending, 16-wide MFMA steps ascending inside a tile) and no split-K.  The
// main tile is BM x BN x BK = 256 x 128 x 64 (eight wave64s of 64 x 64 each);
// launches too small to give it every CU use 128 x 128, 128 x 64 or 64 x 64
// tiles of the same kernel.  A tile only decides which wave computes an element: its row
// and column sit at their index mod 32 inside a 32 x 32 MFMA block under every
// tile, and MFMA rows and columns do not interact.  Rows past M are computed
// from a clamped (valid) row and never stored.  So a row's bits are the same
// for every M, every tile and every position in a tile.
//
// Data path per k-tile: global -> LDS by direct loads (global_load_lds, 16
// bytes per lane, no register staging) into a three-stage ring -> MFMA
// operands.  A [M,K] is stored k-contiguous with a row-dependent XOR swizzle of
// its 16-byte chunks.  W [K,N] stays in its natural n-contiguous layout and
// the B operand, which needs 8 consecutive k per lane, is read with the
// transposing LDS load ds_read_b64_tr_b16 (lane 4a+c of each 16-lane group
// receives column c of the rows its group-mates a, a+4, a+8, a+12 address).
// The LDS serves 32 lanes of an 8-byte read per clock across 64 banks; the W
// layout XORs the 64-byte block of each 256-byte k row with k mod 4, so the
// four k rows a 32-lane half reads fall on four different block positions and
// every transposing read is conflict-free.
//
// Schedule of the 256 x 256 tile: the two wave rows of the workgroup (one
// wave of each per SIMD) take turns, one phase apart: while one reads a
// k-tile's fragments from LDS and issues loads, the other runs its MFMAs on
// the fragments it read in the phase before, at raised issue priority.
// Schedule of the other tiles: one barrier per k-tile, placed before the last
// k-step of k-tile k, publishes k-tile k+1 and frees k-tile k's stage.  Fragments of every
// k-step are read while the previous step's MFMAs run (across the barrier
// too), and the refill loads are issued in small groups after the MFMAs of
// each k-step, so the vector memory unit never holds up a wave that has MFMAs
// to issue.  The ring is unrolled by its depth so that every LDS address is a
// per-thread constant plus an immediate.  Workgroups are placed
// XCD-contiguously and walk groups of 4 row-tiles (row-tiles fastest, then
// columns), so the 32 workgroups resident on one XCD share a 4 x 8 block of A
// rows and W columns in that XCD's L2.
//
// When every tile is the single row-tile (M <= 256), the waves skip the MFMAs
// of their 32-row blocks that hold no row below M, and the A loads that would
// only fill rows past M are not issued: per k-tile one A load (M <= 64), two
// (M <= 128) or all four.  The LDS this frees deepens the ring (6 stages of
// 24 KiB, 4 of 32 KiB, or 3 of 48 KiB), so a small-M launch, which only
// streams W, keeps more of it in flight.  None of this touches a row's
// arithmetic: the same MFMAs in the same k order produce every stored row.
//
// bix_matmul_* is the non-invariant comparator from the problem column of the
// same row: split-K with a split count chosen from the grid size (so from M),
// fp32 partials summed by a second kernel.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace bi {
namespace {

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int STAGES_, int BK_ = kMatmulBK,
          int PP_ = 0, bool ROWSKIP_ = false>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_,
                       STAGES = STAGES_;
  // PP: the two halves of the workgroup take turns (1; 2 also raises the
  // issuing priority of the half in its MFMA phase)
  static constexpr int PP = PP_;
  // ROWSKIP (one 32-row block per wave): a single row-tile launch issues only
  // the A loads that fill rows below M and keeps the ring depth; every wave
  // still runs its MFMAs (a wave whose rows are all past M computes rows that
  // are never stored), so both waves run one instruction stream
  static constexpr bool ROWSKIP = ROWSKIP_;
  static constexpr int NT = 64 * WAVES_M * WAVES_N;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N, MI = WM / 32, NI = WN / 32;
  static constexpr int KS = BK / 16;                  // MFMA k-steps per k-tile
  static constexpr int A_BYTES = BM * BK * 2, W_BYTES = BK * BN * 2, STAGE = A_BYTES + W_BYTES;
  static constexpr int A_LOADS = A_BYTES / 16 / NT;  // 16-byte direct loads per thread
  static constexpr int W_LOADS = W_BYTES / 16 / NT;
  static constexpr int LOADS = A_LOADS + W_LOADS;
  static constexpr int A_ROW = BK * 2, W_ROW = BN * 2;
  static constexpr int A_CPR = BK / 8, W_CPR = BN / 8;  // 16-byte chunks per row
  static constexpr int GROUP_M = 4;                   // row-tiles per raster group
  static_assert(BK == 128 || BK == 64 || BK == 32,
                "A swizzles exist for 256-, 128- and 64-byte rows");
  static_assert(kMatmulBK % BK == 0 || BK == 2 * kMatmulBK,
                "k-tiles divide the k granularity of the interface (or take two of it: such a "
                "tile runs only where k is a multiple of its k-tile)");
  static_assert(BN == 256 || BN == 128 || BN == 64 || BN == 32,
                "W swizzles exist for 32, 16, 8 and 4 chunks per k row");
  static_assert(A_LOADS * NT * 16 == A_BYTES && W_LOADS * NT * 16 == W_BYTES, "tile/threads");
  static_assert(MI * 32 == WM && NI * 32 == WN, "wave tile");
  static_assert(STAGES * STAGE <= 160 * 1024, "LDS");
  static_assert(LOADS <= 63, "vmcnt range");
  // A variant that issues only the first NA of the A loads (single row-tile,
  // M <= 64 NA) keeps NA * 8 KiB of A per stage and deepens the ring to what
  // the same LDS holds: 6 stages for NA = 1, 4 for NA = 2, 3 for NA = 4.
  static constexpr int a_bytes(int na) { return na * NT * 16; }
  static constexpr int stage_bytes(int na) { return a_bytes(na) + W_BYTES; }
  static constexpr int ring(int na) { return ROWSKIP ? STAGES : STAGES * STAGE / stage_bytes(na); }
  // rows of A one load (one per thread) fills
  static constexpr int A_ROWS_PER_LOAD = NT * 16 / A_ROW;
  // the single-row-tile variants (live row blocks, fewer A loads) need two
  // 32-row blocks per wave and A load i filling rows 64i .. 64i+63
  static constexpr bool LIVE_VARIANTS = MI == 2 && A_LOADS == 4 && BM / A_LOADS == 64;
  static_assert(PP == 0 || (!LIVE_VARIANTS && WAVES_M == 2 && WAVES_N == 4 && STAGES >= 3),
                "the alternating halves are the two wave rows");
  static_assert(!ROWSKIP || (MI == 1 && !LIVE_VARIANTS && PP == 0), "row skipping");
};
// The main tile, a larger one for launches with at least a round of them,
// and four smaller ones for launches whose main-tile grid would leave CUs
// idle: 256 x 256 (eight 128 x 64 waves; 32-wide k-tiles, so that four stages
// fit; its wave rows alternate MFMA and memory phases), 128 x 128 (four 64 x 64 waves, one per SIMD), 128 x 64 (four 64 x 32
// waves), 64 x 64 (four 32 x 32 waves) and 64 x 32 (two 32 x 32 waves, twice
// the workgroups on W of a small-M launch).  Where k is a multiple of 128 the
// 64 x 32 tile takes 128-wide k-tiles (half the barriers and waits per byte)
// and, in a single row-tile launch, issues only the A loads of rows below M
// (rows 0..7, 0..15, 0..31 or all 64); a k-tile only groups the same
// ascending 16-wide MFMA steps.
using Tile = TileCfg<256, 128, 4, 2, 3>;
using TileL = TileCfg<256, 256, 2, 4, 4, 32, 2>;
using TileM = TileCfg<128, 128, 2, 2, 3>;
using TileN = TileCfg<128, 64, 2, 2, 4>;
using TileS = TileCfg<64, 64, 2, 2, 4>;
using TileT = TileCfg<64, 32, 2, 1, 6>;
// 64 x 32 with 128-wide k-tiles and row skipping, for k a multiple of 128
using TileTW = TileCfg<64, 32, 2, 1, 6, 128, 0, true>;

// A in LDS: [BM rows][CPR chunks of 16 B]; chunk c of row r sits at
// c ^ swz_a(r).  An MFMA operand read takes one chunk position from each of
// 32 consecutive rows; the 16 lanes the LDS serves together (16 rows, 256 B)
// then fall on 16 different 16-byte bank groups: for 128-byte rows row pairs
// already differ by 128 bytes and the XOR spreads the 8 rows of each parity,
// for 64-byte rows row quads differ by 64 bytes and the XOR spreads the 4
// rows of each residue mod 4, and 256-byte rows, which all start on the same
// bank, are spread by the XOR with r mod 16.
template <int CPR>
__device__ __forceinline__ int swz_a(int r) {
  if constexpr (CPR == 16) return r & 15;
  else if constexpr (CPR == 8) return (r ^ (r >> 3)) & 7;
  else return (r >> 2) & 3;
}
// W in LDS: [BK k rows][CPR chunks of 16 B]; chunk c of k row k sits at
// c ^ swz_w(k), a 64-byte block XOR.  A half-wave's transposing read covers 4
// consecutive k rows (from a multiple of 4) and 64 bytes of each; the XOR
// puts those four 64-byte pieces on four different quarters of the 256-byte
// bank space: by k mod 4 for rows of 256 or 512 bytes (CPR 16, 32), and by
// bit 1 of k for 128-byte rows (CPR 8), whose row pairs already differ by 128
// bytes.
template <int CPR>
__device__ __forceinline__ int swz_w(int k) {
  if constexpr (CPR >= 16) return (k & 3) << 2;
  else if constexpr (CPR == 8) return ((k >> 1) & 1) << 2;
  else return 0;  // 64-byte rows: the four k rows are 256 contiguous bytes
}

// Position of raster id `id` (groups of GROUP_M row-tiles; row-tiles fastest
// inside a group, then columns).
template <class T>
__device__ __forceinline__ void raster_tile(uint32_t id, int tiles_m, int tiles_n, int& m0,
                                            int& n0) {
  const uint32_t per_group = (uint32_t)T::GROUP_M * (uint32_t)tiles_n;
  const int grp = (int)(id / per_group);
  const int grp_rows = min(T::GROUP_M, tiles_m - grp * T::GROUP_M);
  const uint32_t within = id - (uint32_t)grp * per_group;
  m0 = (grp * T::GROUP_M + (int)(within % (uint32_t)grp_rows)) * T::BM;
  n0 = (int)(within / (uint32_t)grp_rows) * T::BN;
}

// Persistent: the invariant launch has about one workgroup per CU.  Workgroup
// b belongs to group x = b mod X (X = min(8, grid); with a grid that is a
// multiple of 8 the groups are the XCDs, which receive workgroups round-robin)
// and the groups own contiguous ranges of the raster order, so a group's
// resident tiles share a block of A and W in its L2.  A workgroup runs its
// tiles back to back through one continuous stream of k-tiles: the ring
// loads the next tile's first k-tiles while the current tile finishes.  The
// split-K comparator launches one workgroup per (tile, slice) instead.
// PW: W comes in the strip layout of bi_matmul_pack_w, [n/32][k][32]: each
// 32-column strip is contiguous along k, so a small-M launch, whose workgroups
// each stream one or two strips, reads whole bursts instead of 64-byte pieces
// of 8 KiB rows.  Only the global addresses differ; what reaches LDS, and so
// every MFMA operand, is the same as with the row-major W.
template <class T, bool SPLIT, bool PW = false>
__global__ __launch_bounds__(T::NT) void bi_matmul_kernel(const uint16_t* __restrict__ A,
                                                             const uint16_t* __restrict__ W,
                                                             void* __restrict__ C, int M, int N,
                                                             int K, int out_f32, int kt_per_split) {
  constexpr int BK = T::BK, NT = T::NT, KS = T::KS, STAGES = T::STAGES;
  constexpr int MI = T::MI, NI = T::NI, STAGE = T::STAGE;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * STAGE];

  const int tiles_m = (M + T::BM - 1) / T::BM;
  const int tiles_n = (N + T::BN - 1) / T::BN;
  const uint32_t ntiles = (uint32_t)tiles_m * (uint32_t)tiles_n;

  // this workgroup's tiles: first, first + step, ... (count of them)
  uint32_t first, step, count;
  int kt0 = 0, kt1 = K / BK;
  if (SPLIT) {
    first = xcd_contiguous_id(blockIdx.x, ntiles);
    step = 1;
    count = 1;
    kt0 = (int)blockIdx.z * kt_per_split;
    kt1 = min(kt1, kt0 + kt_per_split);
  } else {
    const uint32_t G = gridDim.x, X = G < 8 ? G : 8;
    const uint32_t x = blockIdx.x % X, j = blockIdx.x / X;
    const uint32_t gx = G / X + (x < G % X ? 1 : 0);  // workgroups in group x
    const uint32_t q = ntiles / X, r = ntiles % X;
    const uint32_t lo = x * q + (x < r ? x : r), hi = lo + q + (x < r ? 1 : 0);
    first = lo + j;
    step = gx;
    count = first < hi ? (hi - first + step - 1) / step : 0;
  }
  const int nk = kt1 - kt0;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave_m = wave / T::WAVES_N, wave_n = wave % T::WAVES_N;

  // Epilogue: lane holds column (lane & 31) and rows 8*(r/4) + 4*(lane/32) + r%4.
  // bf16 output: the four lanes of a quad hold four adjacent columns of the
  // same four rows.  Two lane exchanges inside the quad (xor 1, then xor 2)
  // transpose that 4x4 block of bf16 values, so that lane q holds row
  // 2(q%2) + q/2 of it, four consecutive columns, stored as one 8-byte write
  // (N is a multiple of 8, so the four columns are all in range or all out).
  const int quad = lane & 3;
  const int quad_row = 2 * (quad & 1) + (quad >> 1);
  auto store_tile_bf16 = [&](int m0, int n0, const f32x16 (&acc)[MI][NI]) __attribute__((always_inline)) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int col = n0 + wave_n * T::WN + ni * 32 + ((lane & 31) & ~3);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t p01 = pack_bf16x2(acc[mi][ni][4 * j], acc[mi][ni][4 * j + 1]);
          const uint32_t p23 = pack_bf16x2(acc[mi][ni][4 * j + 2], acc[mi][ni][4 * j + 3]);
          // xor 1: even lanes keep rows 0,1 and take the odd partner's; odd
          // lanes keep rows 2,3 and take the even partner's
          const uint32_t own = (quad & 1) ? p23 : p01;
          const uint32_t got = (uint32_t)__builtin_amdgcn_mov_dpp((int)((quad & 1) ? p01 : p23),
                                                                  0xB1, 0xF, 0xF, false);
          const uint32_t x = (quad & 1) ? pack_lo(got, own) : pack_lo(own, got);
          const uint32_t y = (quad & 1) ? pack_hi(got, own) : pack_hi(own, got);
          // xor 2: lanes 0,1 keep their first row, lanes 2,3 their second
          const uint32_t got2 =
              (uint32_t)__builtin_amdgcn_mov_dpp((int)((quad & 2) ? x : y), 0x4E, 0xF, 0xF, false);
          const u32x2 v = (quad & 2) ? u32x2{got2, y} : u32x2{x, got2};
          const int row = m0 + wave_m * T::WM + mi * 32 + 8 * j + 4 * (lane >> 5) + quad_row;
          if (row < M && col < N) *(u32x2*)((uint16_t*)C + (int64_t)row * N + col) = v;
        }
      }
    }
  };
  auto store_tile = [&](int m0, int n0, const f32x16 (&acc)[MI][NI]) __attribute__((always_inline)) {
    if (!SPLIT && !out_f32) {
      store_tile_bf16(m0, n0, acc);
      return;
    }
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int col = n0 + wave_n * T::WN + ni * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wave_m * T::WM + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (row < M && col < N) {
            const int64_t o = (int64_t)row * N + col;
            const float v = acc[mi][ni][r];
            if (SPLIT) {
              ((float*)C)[(int64_t)blockIdx.z * M * N + o] = v;
            } else {
              ((float*)C)[o] = v;
            }
          }
        }
      }
    }
  };
  f32x16 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x16{};
  if (nk <= 0) {  // K = 0: every tile is zero
    for (uint32_t t = 0; t < count; ++t) {
      int m0, n0;
      raster_tile<T>(first + t * step, tiles_m, tiles_n, m0, n0);
      store_tile(m0, n0, acc);
    }
    return;
  }

  // ---- the load side: a cursor over the stream of (tile, k-tile) ----------
  // Direct loads: load i of wave w fills the 1 KiB LDS block i*NT/64 + w of
  // the stage's A (or W) part; lane l of it lands at chunk i*NT + 64w + l.
  // Sources are byte offsets from a wave-uniform per-tile base (rows past M
  // clamp to M-1, columns past N to N-8).
  uint32_t a_off[T::A_LOADS], w_off[T::W_LOADS];
  const uint8_t* a_base;
  const uint8_t* w_base;
  auto load_tile = [&](uint32_t t) __attribute__((always_inline)) {
    int m0, n0;
    raster_tile<T>(first + t * step, tiles_m, tiles_n, m0, n0);
#pragma unroll
    for (int i = 0; i < T::A_LOADS; ++i) {
      const int q = i * NT + wave * 64 + lane;
      const int row = q / T::A_CPR, c = (q % T::A_CPR) ^ swz_a<T::A_CPR>(q / T::A_CPR);
      a_off[i] = (uint32_t)(((int64_t)(min(m0 + row, M - 1) - m0) * K + c * 8) * 2);
    }
#pragma unroll
    for (int i = 0; i < T::W_LOADS; ++i) {
      const int q = i * NT + wave * 64 + lane;
      const int k = q / T::W_CPR, c = (q % T::W_CPR) ^ swz_w<T::W_CPR>(q / T::W_CPR);
      const int n = min(n0 + c * 8, N - 8);  // the chunk's first column
      if constexpr (PW)  // strip n/32, row k, column n mod 32 (n0 starts a strip)
        w_off[i] = (uint32_t)((((int64_t)(n / 32 - n0 / 32) * K + k) * 32 + n % 32) * 2);
      else
        w_off[i] = (uint32_t)(((int64_t)k * N + n - n0) * 2);
    }
    a_base = (const uint8_t*)(A + (int64_t)m0 * K);
    w_base = (const uint8_t*)(PW ? W + (int64_t)(n0 / 32) * K * 32 : W + n0);
  };
  const int64_t total = (int64_t)count * nk;  // stream length
  int64_t ipos = 0;                            // stream position of the next load
  uint32_t it = 0;                             // its tile (index into this workgroup's list)
  int ikt = 0;                                 // its k-tile within the tile
  load_tile(0);
  // The cursor stops at the last position: past the end the last k-tile is
  // loaded again into a stage nobody reads, so every k-tile issues exactly
  // one tile of loads and vmcnt counts stay exact.
  auto advance = [&]() __attribute__((always_inline)) {
    if (ipos + 1 < total) {
      ++ipos;
      if (++ikt == nk) {
        ikt = 0;
        load_tile(++it);
      }
    }
  };
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  // loads [lo, hi) of the cursor's k-tile into `stage`: the first NA A loads
  // (load i fills A rows 64i .. 64i+63 of the stage), then the W loads.
  auto issue = [&](int stage, int lo, int hi, auto nc) __attribute__((always_inline)) {
    constexpr int NA = decltype(nc)::value;
    const int kt = kt0 + ikt;
    const uint8_t* ab = a_base + (int64_t)kt * (BK * 2);
    // elements from one k row of W to the next: 32 in a strip, else N
    const uint8_t* wb = w_base + (int64_t)kt * BK * (PW ? 32 : N) * 2;
    const uint32_t sb = lds0 + stage * T::stage_bytes(NA) + wave * 1024;
#pragma unroll
    for (int i = 0; i < NA; ++i)
      if (i >= lo && i < hi) lds_dma16_sv(ab, a_off[i], sb + i * NT * 16);
#pragma unroll
    for (int i = 0; i < T::W_LOADS; ++i)
      if (NA + i >= lo && NA + i < hi)
        lds_dma16_sv(wb, w_off[i], sb + T::a_bytes(NA) + i * NT * 16);
  };

  // Per-thread LDS read offsets within a stage.
  // A operand of k-step kk, block mi: row r = wave_m*64 + 32mi + l%32,
  // k = 16kk + 8(l/32) .. +7.
  uint32_t ao[KS][MI];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk)
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int r = wave_m * T::WM + mi * 32 + (lane & 31);
      const int ch = 2 * kk + (lane >> 5);
      ao[kk][mi] = (uint32_t)(r * T::A_ROW + ((ch ^ swz_a<T::A_CPR>(r)) << 4));
    }
  // B operand, block ni: lane l needs W[16kk + 8(l/32) + e][col + l%32],
  // e = 0..7, as two transposed reads of 4 k rows; within a 16-lane group,
  // lane i addresses k row base + i/4, columns 4(i%4)..+3 of the group's 16.
  const int g16 = lane >> 4, i16 = lane & 15;
  uint32_t wo[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    const int nb = wave_n * T::WN + ni * 32 + 16 * (g16 & 1) + 4 * (i16 & 3);
    const int k = 8 * (g16 >> 1) + (i16 >> 2);
    wo[ni] = (uint32_t)(k * T::W_ROW + (((nb >> 3) ^ swz_w<T::W_CPR>(k)) << 4) + (nb & 7) * 2);
  }

  // fragments of k-step kk from the stage at S: the first NB row blocks of A
  // and all of B (whose part starts after the variant's NA A loads)
  auto frags_n = [&](const uint8_t* S, int kk, bf16x8 (&af)[MI], bf16x8 (&bw)[NI], auto nb,
                     auto nc) __attribute__((always_inline)) {
    constexpr int NB = decltype(nb)::value, NA = decltype(nc)::value;
#pragma unroll
    for (int mi = 0; mi < NB; ++mi) af[mi] = as_bf16x8(*(const u32x4*)(S + ao[kk][mi]));
    const uint8_t* Sw = S + T::a_bytes(NA);
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      s16x4 v[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
        v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(Sw + wo[ni] + (16 * kk + 4 * h) * T::W_ROW));
      bw[ni] = join_tr(v[0], v[1]);
    }
  };

  // ---- the compute side ------------------------------------------------
  uint32_t ct = 0;  // tile being accumulated
  int ckt = 0;      // its k-tiles done
  int cm0, cn0;
  raster_tile<T>(first, tiles_m, tiles_n, cm0, cn0);
  // One k-tile j held in stage S.  Its step-0 fragments were read during the
  // previous k-tile's last step.  Steps 0..KS-2 read the next step's
  // fragments under their MFMAs and issue load groups 1.. of k-tile j+2 (into
  // the stage of j-1, free since the barrier before j-1's last step).  Before
  // the last step every wave waits for its own loads of k-tile j+1; the
  // barrier publishes it and ends every read of stage S, so the last step's
  // MFMAs run under the reads of j+1's step 0, and group 0 of k-tile j+3 goes
  // out into stage S at once.
  bf16x8 fa[2][MI], fb[2][NI];
  auto issue_group = [&](int stage, int g, auto nc) __attribute__((always_inline)) {
    constexpr int LOADS = decltype(nc)::value + T::W_LOADS;
    constexpr int GRP = (LOADS + KS - 1) / KS;  // loads per group
    issue(stage, g * GRP, min((g + 1) * GRP, LOADS), nc);
  };
  // Rows past M are never stored, and MFMA rows do not interact, so when every
  // tile is the single row-tile (M <= BM), the MFMAs (and A reads) of a wave's
  // 32-row blocks that hold no row below M are skipped: the kernel runs the
  // variant with this wave's LIVE blocks throughout.  A row's bits stay those
  // of the full tile (same instruction, same k order); at small M the tile
  // then streams W instead of computing padding.
  // In the same case the A loads that would fill only rows past M are not
  // issued either: NA = 1 (M <= 64), 2 (M <= 128) or all 4 A loads per k-tile.
  // Every row an MFMA of a live block reads lies below 64 * ceil(M / 64).
  int live = MI, na = T::A_LOADS;
  if (T::ROWSKIP && tiles_m == 1) {
    // the A loads cover the first ceil(M / rows per load) row groups, rounded
    // up to 1, 2, 4 or all of them
    const int need = (M + T::A_ROWS_PER_LOAD - 1) / T::A_ROWS_PER_LOAD;
    na = need <= 1 ? 1 : (need <= 2 ? 2 : (need <= 4 ? 4 : T::A_LOADS));
  }
  if (T::LIVE_VARIANTS && tiles_m == 1) {
    const int rows = M - wave_m * T::WM;
    live = __builtin_amdgcn_readfirstlane(rows <= 0 ? 0 : (rows >= MI * 32 ? MI : (rows + 31) / 32));
    na = M <= 64 ? 1 : (M <= 128 ? 2 : T::A_LOADS);
  }
  // the fragments of step kk for the first LIVE row blocks (all of B if any)
  auto frags_live = [&](const uint8_t* S, int kk, bf16x8 (&af)[MI], bf16x8 (&bw)[NI],
                        auto lc, auto nc) __attribute__((always_inline)) {
    if constexpr (decltype(lc)::value > 0) frags_n(S, kk, af, bw, lc, nc);
  };
  // One k-tile in stage S of a ring of R = ring(NA) stages.
  auto ktile_body = [&](auto sc, auto lc, auto nc) __attribute__((always_inline)) {
    constexpr int S = decltype(sc)::value, LIVE = decltype(lc)::value;
    constexpr int NA = decltype(nc)::value, LOADS = NA + T::W_LOADS, R = T::ring(NA);
    constexpr int SB = T::stage_bytes(NA);
    const uint8_t* Sp = smem + S * SB;
    const uint8_t* Snext = smem + ((S + 1) % R) * SB;
    constexpr int sn = (S + R - 1) % R;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      __builtin_amdgcn_sched_barrier(0);
      if (kk + 1 < KS) {
        frags_live(Sp, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1], lc, nc);
      } else {
        wait_vmcnt_le<(R - 2) * LOADS>();
        __syncthreads();  // next k-tile visible; every wave is done with this stage
        __builtin_amdgcn_sched_barrier(0);
        // all of them: the next k-tile may start a tile with more live rows
        frags_n(Snext, 0, fa[(kk + 1) & 1], fb[(kk + 1) & 1], std::integral_constant<int, MI>{},
                nc);
      }
#pragma unroll
      for (int mi = 0; mi < LIVE; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni] = mfma32(fa[kk & 1][mi], fb[kk & 1][ni], acc[mi][ni]);
      // the next reads interleaved one for one with this step's MFMAs
#pragma unroll
      for (int i = 0; i < LIVE * NI; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      }
      __builtin_amdgcn_sched_barrier(0);
      if (kk + 1 < KS) {
        issue_group(sn, kk + 1, nc);
        if (kk + 2 == KS) advance();
      } else {
        issue_group(S, 0, nc);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto ktile = [&](auto sc, auto lc, auto nc) __attribute__((always_inline)) {
    ktile_body(sc, lc, nc);
    if (++ckt == nk) {  // the tile is complete
      store_tile(cm0, cn0, acc);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x16{};
      ckt = 0;
      if (++ct < count) raster_tile<T>(first + ct * step, tiles_m, tiles_n, cm0, cn0);
    }
  };
  if (count == 0) return;
  // The main loop is unrolled by the ring depth, so every stage offset is an
  // immediate.
  auto run = [&](auto lc, auto nc) __attribute__((always_inline)) {
    constexpr int NA = decltype(nc)::value, LOADS = NA + T::W_LOADS, R = T::ring(NA);
    static_assert(R >= 3 && R * T::stage_bytes(NA) <= STAGES * STAGE, "ring");
    static_assert((R - 2) * LOADS <= 63, "vmcnt range");
#pragma unroll
    for (int s = 0; s < R - 1; ++s) {
      issue(s, 0, LOADS, nc);
      advance();
    }
    // the first k-tile: wait for it, publish it, read its step 0; the last
    // stage is free, so group 0 of k-tile R-1 goes out
    wait_vmcnt_le<(R - 2) * LOADS>();
    __syncthreads();
    frags_n(smem, 0, fa[0], fb[0], std::integral_constant<int, MI>{}, nc);
    issue_group(R - 1, 0, nc);
    int64_t p = 0;
    for (; p + R <= total; p += R)
      static_for<0, R>([&](auto sc) __attribute__((always_inline)) { ktile(sc, lc, nc); });
    static_for<0, R - 1>([&](auto sc) __attribute__((always_inline)) {
      if (p + decltype(sc)::value < total) ktile(sc, lc, nc);
    });
  };
  // one variant for the whole launch: (live blocks of this wave, A loads)
  auto run_live = [&](auto nc) __attribute__((always_inline)) {
    if (!(T::LIVE_VARIANTS || T::ROWSKIP) || live == MI)
      run(std::integral_constant<int, MI>{}, nc);
    else if constexpr (T::LIVE_VARIANTS || T::ROWSKIP) {
      if (live == 1)
        run(std::integral_constant<int, 1>{}, nc);
      else
        run(std::integral_constant<int, 0>{}, nc);
    }
  };
  // Alternating halves (T::PP).  Wave w runs on SIMD w mod 4, so each SIMD
  // holds one wave of each wave row: half 0 (rows 0..BM/2-1) and half 1.  A
  // wave alternates a memory phase (read the whole k-tile's fragments, issue
  // its loads of the k-tile R-1 ahead) and an MFMA phase on those fragments,
  // one barrier after each; half 1 runs one phase behind half 0, so while one
  // wave of a SIMD issues its MFMAs the other reads LDS and loads.  Phase
  // slots: half 0 reads k-tile j in slot 2j-1 and multiplies in 2j; half 1
  // reads in 2j and multiplies in 2j+1.  So k-tile j's stage is free from slot
  // 2j+1, when the loads of k-tile j+R-1 go out into it (half 0 in 2j+1, half
  // 1 in 2j+2), and each wave waits for its own loads of k-tile j+1 before the
  // barrier that ends slot 2j (half 0 after its MFMA phase, half 1 after its
  // memory phase): R-2 later k-tiles of its loads may still be in flight.
  // Every element sees the same MFMAs in the same k order as in the other
  // tiles; only the issue order across the halves changes.
  auto run_pp = [&]() __attribute__((always_inline)) {
    constexpr int NA = T::A_LOADS, LOADS = NA + T::W_LOADS, R = STAGES;
    static_assert((R - 2) * LOADS <= 63, "vmcnt range");
    constexpr auto nc = std::integral_constant<int, NA>{};
    constexpr auto all = std::integral_constant<int, MI>{};
    const bool half1 = wave_m != 0;
    bf16x8 pa[KS][MI], pb[KS][NI];
    auto slot_pair = [&](auto sc) __attribute__((always_inline)) {
      constexpr int S = decltype(sc)::value;
      // memory phase
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) frags_n(smem + S * STAGE, kk, pa[kk], pb[kk], all, nc);
      issue((S + R - 1) % R, 0, LOADS, nc);
      advance();
      if (half1) wait_vmcnt_le<(R - 2) * LOADS>();
      lds_reads_done();
      __syncthreads();
      // MFMA phase
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (T::PP == 2) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = mfma32(pa[kk][mi], pb[kk][ni], acc[mi][ni]);
      if constexpr (T::PP == 2) __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
      if (++ckt == nk) {  // the tile is complete
        store_tile(cm0, cn0, acc);
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x16{};
        ckt = 0;
        if (++ct < count) raster_tile<T>(first + ct * step, tiles_m, tiles_n, cm0, cn0);
      }
      if (!half1) wait_vmcnt_le<(R - 2) * LOADS>();
      __syncthreads();
    };
#pragma unroll
    for (int s = 0; s < R - 1; ++s) {
      issue(s, 0, LOADS, nc);
      advance();
    }
    wait_vmcnt_le<(R - 2) * LOADS>();
    __syncthreads();
    if (half1) __syncthreads();  // half 1 starts one phase behind
    int64_t p = 0;
    for (; p + R <= total; p += R) static_for<0, R>(slot_pair);
    static_for<0, R - 1>([&](auto sc) __attribute__((always_inline)) {
      if (p + decltype(sc)::value < total) slot_pair(sc);
    });
    if (!half1) __syncthreads();  // as many barriers as half 1
  };
  if constexpr (T::PP != 0 && !SPLIT) {
    run_pp();
  } else if constexpr (T::ROWSKIP && !SPLIT) {
    constexpr int NA4 = T::A_LOADS > 4 ? 4 : T::A_LOADS;
    if (na == 1)
      run_live(std::integral_constant<int, 1>{});
    else if (na == 2)
      run_live(std::integral_constant<int, 2>{});
    else if (na == 4)
      run_live(std::integral_constant<int, NA4>{});
    else
      run_live(std::integral_constant<int, T::A_LOADS>{});
  } else if constexpr (SPLIT || !T::LIVE_VARIANTS) {  // the comparator keeps the one full ring
    run_live(std::integral_constant<int, T::A_LOADS>{});
  } else {
    if (na == 1)
      run_live(std::integral_constant<int, 1>{});
    else if (na == 2)
      run_live(std::integral_constant<int, 2>{});
    else
      run_live(std::integral_constant<int, T::A_LOADS>{});
  }
  wait_vmcnt_le<0>();  // no LDS write may outlive the workgroup
}

// W [k, n] row-major -> the strip layout [n/32][k][32]; one 16-byte chunk
// (8 columns) per thread, read along W's rows.
__global__ __launch_bounds__(256) void bi_matmul_pack_w_kernel(const uint16_t* __restrict__ w,
                                                                uint16_t* __restrict__ wp,
                                                                int64_t k, int64_t n) {
  const int64_t chunks = k * (n / 8);
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= chunks) return;
  const int64_t row = i / (n / 8), c8 = i % (n / 8);
  const u32x4 v = *(const u32x4*)(w + row * n + c8 * 8);
  *(u32x4*)(wp + ((c8 / 4) * k + row) * 32 + (c8 % 4) * 8) = v;
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

// Compute units of the current device (one persistent workgroup each), asked
// once per device and kept for the process (256, the MI355X count, if the
// runtime cannot say).
int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices] = {};
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < kMaxDevices) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < kMaxDevices) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

template <class T>
static int64_t tile_count(int64_t m, int64_t n) {
  return ((m + T::BM - 1) / T::BM) * ((n + T::BN - 1) / T::BN);
}

// The tile: the first of 64 x 32, 64 x 64, 128 x 64 and 128 x 128 whose tiles
// number at most one per CU; else, with several row-tiles, 256 x 256 where its
// rounds of tiles are estimated to finish first, else the main tile (both
// persistent, at most one workgroup per CU).  A smaller tile moves more bytes
// per flop from L2 to LDS, and the smaller tiles run one wave per SIMD; so
// past one round of tiles the larger tiles' fewer, denser tiles finish first.
// All six run the same MFMA instruction on the same operands in the same k order
// for every output element (a row or column's place inside a 32 x 32 block is
// its index mod 32 under each tile, and the k-tile width only groups the same
// ascending 16-wide steps), so the choice changes no bits.
template <class T>
static void launch_tile(const void* a, const void* w, void* c, bool c_f32, int64_t m, int64_t n,
                        int64_t k, int64_t grid, bool packed, hipStream_t st) {
  if (packed)
    hipLaunchKernelGGL((bi_matmul_kernel<T, false, true>), dim3((unsigned)grid), dim3(T::NT), 0,
                       st, (const uint16_t*)a, (const uint16_t*)w, c, (int)m, (int)n, (int)k,
                       c_f32 ? 1 : 0, 0);
  else
    hipLaunchKernelGGL((bi_matmul_kernel<T, false>), dim3((unsigned)grid), dim3(T::NT), 0, st,
                       (const uint16_t*)a, (const uint16_t*)w, c, (int)m, (int)n, (int)k,
                       c_f32 ? 1 : 0, 0);
}

void matmul_tile(int64_t m, int64_t n, int* bm, int* bn, int64_t* grid) {
  const int64_t cus = device_cus();
  const int64_t ts = tile_count<TileS>(m, n), tn = tile_count<TileN>(m, n);
  const int64_t tm = tile_count<TileM>(m, n), tq = tile_count<TileT>(m, n);
  if (tq <= cus) {
    *bm = TileT::BM, *bn = TileT::BN, *grid = tq;
  } else if (ts <= cus) {
    *bm = TileS::BM, *bn = TileS::BN, *grid = ts;
  } else if (tn <= cus) {
    *bm = TileN::BM, *bn = TileN::BN, *grid = tn;
  } else if (tm <= cus) {
    *bm = TileM::BM, *bn = TileM::BN, *grid = tm;
  } else {
    // persistent: each CU runs ceil(tiles / CUs) tiles back to back, and a
    // 256 x 256 tile takes about 1.6 times a 256 x 128 one (measured at
    // 2048 x 4096 x 14336: 93 against 59 us per tile)
    const int64_t tl = tile_count<TileL>(m, n), tt = tile_count<Tile>(m, n);
    if (m > TileL::BM && 8 * ((tl + cus - 1) / cus) < 5 * ((tt + cus - 1) / cus)) {
      *bm = TileL::BM, *bn = TileL::BN, *grid = std::min(tl, cus);
    } else {
      *bm = Tile::BM, *bn = Tile::BN, *grid = std::min(tt, cus);
    }
  }
}

hipError_t launch_matmul(const void* a, const void* w, void* c, bool c_f32, int64_t m, int64_t n,
                         int64_t k, hipStream_t st, bool packed) {
  int bm, bn;
  int64_t grid;
  matmul_tile(m, n, &bm, &bn, &grid);
  if (bm == TileT::BM && bn == TileT::BN && k % TileTW::BK == 0)
    launch_tile<TileTW>(a, w, c, c_f32, m, n, k, grid, packed, st);
  else if (bm == TileT::BM && bn == TileT::BN)
    launch_tile<TileT>(a, w, c, c_f32, m, n, k, grid, packed, st);
  else if (bm == TileS::BM)
    launch_tile<TileS>(a, w, c, c_f32, m, n, k, grid, packed, st);
  else if (bm == TileN::BM && bn == TileN::BN)
    launch_tile<TileN>(a, w, c, c_f32, m, n, k, grid, packed, st);
  else if (bm == TileM::BM)
    launch_tile<TileM>(a, w, c, c_f32, m, n, k, grid, packed, st);
  else if (bn == TileL::BN)
    launch_tile<TileL>(a, w, c, c_f32, m, n, k, grid, packed, st);
  else
    launch_tile<Tile>(a, w, c, c_f32, m, n, k, grid, packed, st);
  return hipGetLastError();
}

hipError_t launch_matmul_pack_w(const void* w, void* wp, int64_t k, int64_t n, hipStream_t st) {
  const int64_t chunks = k * (n / 8);
  if (chunks > 0)
    hipLaunchKernelGGL(bi_matmul_pack_w_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256),
                       0, st, (const uint16_t*)w, (uint16_t*)wp, k, n);
  return hipGetLastError();
}

// The comparator takes bi_matmul's tile for the shape and splits k only to
// fill CUs that tile leaves idle (the usual split-K heuristic): enough slices
// for one workgroup per CU, at most 16 and at most one k-tile each.  With one
// slice it is bi_matmul itself.
int matmul_splitk_auto(int64_t m, int64_t n, int64_t k) {
  int bm, bn;
  int64_t grid;
  matmul_tile(m, n, &bm, &bn, &grid);
  const int64_t tiles = ((m + bm - 1) / bm) * ((n + bn - 1) / bn);
  int64_t s = (device_cus() + tiles - 1) / (tiles > 0 ? tiles : 1);
  const int64_t kt = k / Tile::BK;
  if (s > 16) s = 16;
  if (s > kt) s = kt;
  if (s < 1) s = 1;
  return (int)s;
}

// k cut into split_k slices of whole k-tiles of the tile's width; returns the
// slices that own at least one k-tile (at most split_k).
template <class T>
static int launch_split(const void* a, const void* w, float* ws, int64_t m, int64_t n,
                        int split_k, int64_t k, bool packed, hipStream_t st) {
  const int kt = (int)(k / T::BK);
  const int per = (kt + split_k - 1) / split_k;
  const int used = (kt + per - 1) / per;
  const int64_t tiles = tile_count<T>(m, n);
  if (packed)
    hipLaunchKernelGGL((bi_matmul_kernel<T, true, true>), dim3((unsigned)tiles, 1, (unsigned)used),
                       dim3(T::NT), 0, st, (const uint16_t*)a, (const uint16_t*)w, (void*)ws,
                       (int)m, (int)n, (int)k, 1, per);
  else
    hipLaunchKernelGGL((bi_matmul_kernel<T, true>), dim3((unsigned)tiles, 1, (unsigned)used),
                       dim3(T::NT), 0, st, (const uint16_t*)a, (const uint16_t*)w, (void*)ws,
                       (int)m, (int)n, (int)k, 1, per);
  return used;
}

hipError_t launch_matmul_splitk(const void* a, const void* w, void* c, bool c_f32, int64_t m,
                                int64_t n, int64_t k, int split_k, float* ws, hipStream_t st,
                                bool packed) {
  if (split_k <= 1) return launch_matmul(a, w, c, c_f32, m, n, k, st, packed);
  int bm, bn;
  int64_t grid;
  matmul_tile(m, n, &bm, &bn, &grid);
  int used;
  if (bm == TileT::BM && bn == TileT::BN)
    used = launch_split<TileT>(a, w, ws, m, n, split_k, k, packed, st);
  else if (bm == TileS::BM)
    used = launch_split<TileS>(a, w, ws, m, n, split_k, k, packed, st);
  else if (bm == TileN::BM && bn == TileN::BN)
    used = launch_split<TileN>(a, w, ws, m, n, split_k, k, packed, st);
  else if (bm == TileM::BM)
    used = launch_split<TileM>(a, w, ws, m, n, split_k, k, packed, st);
  else  // 256 x 256 (whose one-slice launch has no registers to spare) or the main tile
    used = launch_split<Tile>(a, w, ws, m, n, split_k, k, packed, st);
  const int64_t count = m * n;
  hipLaunchKernelGGL(bix_matmul_reduce_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0,
                     st, (const float*)ws, c, count, used, c_f32 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace bi
