// Paged split-KV attention: append, split partials, fixed-order fold.
//
// Follows the Attention row of the approach table in "Defeating
// Nondeterminism in LLM Inference" (mobiles-han.blogspot.com summary):
//   * one unified layout -- a call first appends its new keys/values to the
//     paged pool (kv_append_kernel); attention then reads the pool only, so a
//     token's keys take the same path whether they arrived in this call or
//     long ago;
//   * fixed-size splits -- keys are cut at absolute multiples of 256.  The
//     partial of one split for one query column is computed by ONE pair of
//     device functions (split_qk, then split_pv), and partials are folded left
//     in ascending split order by ONE pair of device functions (fold_coef,
//     fold_apply).  Prefill folds in registers; decode writes partials to a
//     workspace and a second kernel folds them; both run the same functions on
//     the same operand values, so a token's output row has the same bits
//     either way.  Operands always come from LDS with the same layout; only
//     how they get there differs: decode streams each wave's units through a
//     wave-private ring of 8 chunk slots (StreamSrc; 4 for the int16 cache),
//     prefill copies a whole split into LDS for the waves of a workgroup to
//     share (StagedSrc), and the split-count comparator streams each split
//     through a ring of 5 slots (RingSrc).  All copy with direct global->LDS
//     loads whose page is wave-uniform.  (bf16 decode appends inside its split
//     pass: the one wave that reads a sequence's last split for a kv head
//     stores the new rows before it loads them.)
//
// Work unit: one wave64 computes the partial of one split for NB blocks of 16
// query columns (GQA: the columns of a block are (position, head-of-group)
// pairs sharing one kv head) with v_mfma_f32_16x16x32_bf16:
//   S^T = K Q^T   (A = 16 keys x 32 dims, B = Q^T held in registers)
//   O^T = V^T P^T (A = 16 dims x 32 keys, B = P^T straight from registers)
// Keys of a 32-key chunk are permuted onto MFMA rows so that each lane's
// accumulator holds the 8 consecutive keys it needs as the P^T operand; the
// V^T operand is read from LDS with the transposing load ds_read_b64_tr_b16.
// All 8 chunks of a split that starts at or before a column's position are
// computed (a split wholly past every column of a wave is never visited).
// Keys beyond a column's position get logit -inf and weight exactly 0, and
// their addresses are clamped to the last written position, so they add exact
// zeros: a split's bits do not depend on how far past the query the split's
// keys run.
//
// bix_attn_decode_splitkv_* is the comparator from the problem column of the
// same row: the key range of each sequence is cut into a number of splits
// chosen from the batch, so split boundaries move with the batch.
#include <limits.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace bi {
namespace {

constexpr float kLn2 = 0.693147180559945309f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// One step of the left fold:  m' = max(m, ms); l = l e^(m-m') + ls e^(ms-m'),
// o = o e^(m-m') + os e^(ms-m') (base-2 logits, so e^ is exp2; the first
// product is fused into the add).
struct FoldCoef {
  float a, b, m;
};
__device__ __forceinline__ FoldCoef fold_coef(float m, float ms) {
  const float mn = fmaxf(m, ms);
  return FoldCoef{fast_exp2(m - mn), fast_exp2(ms - mn), mn};
}
__device__ __forceinline__ float fold_apply(float x, float xs, const FoldCoef& f) {
  return fmaf(x, f.a, xs * f.b);
}
// Natural-log lse from base-2 max and sum.
__device__ __forceinline__ float lse_of(float m2, float l) { return (m2 + fast_log2(l)) * kLn2; }

template <int D>
struct KV {
  static constexpr int DS = D / 32;    // 32-wide MFMA k-steps over the head dim
  static constexpr int DB = D / 16;    // O^T row blocks; lane owns DB consecutive dims
  static constexpr int ROWB = D * 2;   // bytes per key row
  static constexpr int CPR = D / 8;    // 16-byte chunks per key row
  using vrow = std::conditional_t<D == 128, u32x4, u32x2>;  // DB dims of one key
};

// In-chunk key of the S^T A-operand row this lane loads for half h.
__device__ __forceinline__ int okey_k(int h, int r) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Key rows in LDS are D*2 bytes; their 16-byte chunks are XOR-swizzled by key
// (k = key index within a 32-key chunk).  The LDS has 64 banks of 4 bytes and
// serves 16 lanes of a 16-byte read, or 32 lanes of an 8-byte read, per clock.
// K: chunk c of key k sits at c ^ kswz(k).  One clock of an S^T operand read
// covers 16 keys that differ in bits 0, 1, 3, 4 of k; kswz maps them to 16
// distinct 16-byte slots of the 256-byte bank row (d=128), or to 8 distinct
// slots in each half for the two keys sharing a bank row (d=64).
// V: chunk c sits at c ^ vswz(k).  One clock of a transposed read covers 8
// keys (bits 0, 1, 3) x 32 bytes; vswz gives each key a distinct 32-byte slot.
template <int D>
__device__ __forceinline__ int kswz(int k) {
  if constexpr (D == 128) return (k & 3) | (((k >> 3) & 3) << 2);
  else return ((k >> 1) & 1) | (((k >> 3) & 3) << 1);
}
template <int D>
__device__ __forceinline__ int vswz(int k) {
  if constexpr (D == 128) return ((k & 3) << 1) | (((k >> 3) & 1) << 3);
  else return (((k >> 1) & 1) | (((k >> 3) & 1) << 1)) << 1;
}

// ---- operand source: keys and values of 32-key chunks held in LDS ---------------
// load_k<C>(kb): kb[h][t] = K[32C+okey_k(h,r)][32t+8q .. +7] of the split
// load_v<C>(va): va[i]    = V[32C+8q .. 32C+8q+7][16i+r] (one bf16x8 per lane),
//                read with two transposing loads (ds_read_b64_tr_b16): within
//                each 16-lane group, lane i' addresses key 8q+4hh+i'/4, dims
//                16i+4(i'%4)..+3, and lane j receives dim 16i+j of the 4 keys.
// step<IDX>() runs before chunk IDX (0..7: K chunks, 8..15: V chunks) so a
// source that streams chunks can wait for / refill its buffers.
template <int D>
__device__ __forceinline__ u32x4 lds_k_operand(const uint8_t* rows, int h, int t) {
  const int lane = threadIdx.x & (kWave - 1), r = lane & 15, q = lane >> 4;
  const int k = okey_k(h, r);
  return *(const u32x4*)(rows + k * KV<D>::ROWB + (((4 * t + q) ^ kswz<D>(k)) << 4));
}
template <int D>
__device__ __forceinline__ bf16x8 lds_v_operand(const uint8_t* rows, int i) {
  const int lane = threadIdx.x & (kWave - 1), r = lane & 15, q = lane >> 4;
  const int d = 16 * i + 4 * (r & 3);
  s16x4 v[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int k = 8 * q + 4 * hh + (r >> 2);
    const uint8_t* p = rows + k * KV<D>::ROWB + (((d >> 3) ^ vswz<D>(k)) << 4) + (d & 7) * 2;
    v[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  }
  return join_tr(v[0], v[1]);
}

// Page numbers of one 256-key split: pg[i] holds positions key0+16i..+15;
// entries past the last written position use that position's page.  All
// wave-uniform (scalar registers).
struct SplitPages {
  int pg[16];
  __device__ __forceinline__ void load(const int32_t* bt_row, int key0, int last) {
    if (key0 + 255 <= last) {
      // a fully written split: 16 consecutive block-table entries
      const int32_t* row = bt_row + (key0 >> 4);
#pragma unroll
      for (int i = 0; i < 16; ++i) pg[i] = __builtin_amdgcn_readfirstlane(row[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        pg[i] = __builtin_amdgcn_readfirstlane(bt_row[min(key0 + 16 * i, last) >> 4]);
    }
  }
};

// Start of the (page, kv head) block of a pool whose kv-head-g base is
// pool_g: pages are page_elems = nkv*16*D elements apart (a 32 x 32 -> 64-bit
// product of bytes).
__device__ __forceinline__ const uint16_t* page_block(const uint16_t* pool_g, int page,
                                                      uint32_t page_elems) {
  return (const uint16_t*)((const uint8_t*)pool_g + (uint64_t)(uint32_t)page * (2u * page_elems));
}

// Byte offset, inside one (page, kv head) block, of the 16-byte chunk a lane
// of a direct load fetches for split key kl = kfirst + lane/CPR when no
// clamping is needed: row kl mod 16, logical chunk phys ^ swz(kl).  Only kl
// mod 32 matters, so a load's offsets depend on kfirst mod 32 alone and can be
// computed once per kernel.
template <int D, bool IS_K>
__device__ __forceinline__ uint32_t dma_lane_off(int kfirst) {
  constexpr int CPR = KV<D>::CPR;
  const int lane = threadIdx.x & (kWave - 1);
  const int kl = kfirst + lane / CPR, phys = lane % CPR;
  const int logical = phys ^ (IS_K ? kswz<D>(kl) : vswz<D>(kl));
  return (uint32_t)(((kl & 15) * D + logical * 8) * 2);
}

// One direct 1 KiB global->LDS load of the rows of keys kfirst..kfirst+KPI-1
// of a split (KPI = 64 / chunks per row; all in the uniform page `page`) of
// one kv head, swizzled for K or V, to LDS address lds_block.  Keys past
// `last` read key `last` instead, so every value loaded is a written one.
template <int D, bool IS_K, bool STREAM = false>
__device__ __forceinline__ void dma_block(const uint16_t* pool, int page, int nkv, int g, int key0,
                                          int kfirst, int last, uint32_t lds_block) {
  constexpr int CPR = KV<D>::CPR;
  const int lane = threadIdx.x & (kWave - 1);
  const int kl = kfirst + lane / CPR, phys = lane % CPR;
  const int logical = phys ^ (IS_K ? kswz<D>(kl) : vswz<D>(kl));
  // past the last position the page is already last's (SplitPages), so only
  // the slot needs clamping
  const int slot = min(key0 + kl, last) & 15;
  const uint16_t* base = pool + ((int64_t)page * nkv + g) * 16 * D;
  lds_dma16_sv<STREAM>(base, (uint32_t)(slot * D + logical * 8) * 2, lds_block);
}

// LDS addresses of this lane's operand reads in chunk 0 of a K / V region
// (the same addressing as lds_k_operand / lds_v_operand), so that a read of
// chunk C is one LDS load with an immediate offset.
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
template <int D>
struct OperandLanes {
  uint32_t k[2][KV<D>::DS];  // (half h, d-step t)
  uint32_t v[KV<D>::DB][2];  // (dim block i, key half hh)
  __device__ __forceinline__ void init(uint32_t kregion, uint32_t vregion) {
    const int lane = threadIdx.x & (kWave - 1), r = lane & 15, q = lane >> 4;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int t = 0; t < KV<D>::DS; ++t) {
        const int kk = okey_k(h, r);
        k[h][t] = kregion + kk * KV<D>::ROWB + (((4 * t + q) ^ kswz<D>(kk)) << 4);
      }
#pragma unroll
    for (int i = 0; i < KV<D>::DB; ++i)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int d = 16 * i + 4 * (r & 3), kk = 8 * q + 4 * hh + (r >> 2);
        v[i][hh] = vregion + kk * KV<D>::ROWB + (((d >> 3) ^ vswz<D>(kk)) << 4) + (d & 7) * 2;
      }
  }
};

// A whole split staged in LDS by the workgroup (prefill): K and V rows of
// keys 0..255 at the regions OperandLanes was built for.
template <int D>
struct StagedSrc {
  OperandLanes<D> ol;
  template <int IDX>
  __device__ __forceinline__ void step() const {}
  template <int C>
  __device__ __forceinline__ u32x4 k(int h, int t) const {
    return *(lds_u32x4*)(uintptr_t)(ol.k[h][t] + 32 * C * KV<D>::ROWB);
  }
  template <int C>
  __device__ __forceinline__ bf16x8 v(int i) const {
    s16x4 x[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      x[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)(uintptr_t)(ol.v[i][hh] + 32 * C * KV<D>::ROWB));
    return join_tr(x[0], x[1]);
  }
};

// The same over the int16 cache: the operands are int16, and the split's 256
// key and value dequantisation factors sit in LDS (kscl, vscl).  kscale<C> /
// vscale(C) give this lane's keys 32C + 8q .. +7.
typedef __attribute__((address_space(3))) const f32x4 lds_f32x4;
template <int D>
struct StagedSrc16 : StagedSrc<D> {
  static constexpr bool Q16 = true;
  uint32_t kscl, vscl;
  __device__ __forceinline__ void factors(uint32_t base, int C, float (&f)[8]) const {
    const int q = (threadIdx.x & (kWave - 1)) >> 4;
    const uint32_t a = base + (uint32_t)(32 * C + 8 * q) * 4;
    const f32x4 x = *(lds_f32x4*)(uintptr_t)a, y = *(lds_f32x4*)(uintptr_t)(a + 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[j] = x[j];
      f[4 + j] = y[j];
    }
  }
  __device__ __forceinline__ void kscale(int C, float (&f)[8]) const { factors(kscl, C, f); }
  __device__ __forceinline__ void vscale(int C, float (&f)[8]) const { factors(vscl, C, f); }
};

// A split streamed chunk by chunk through a wave-private ring of RING LDS
// slots (decode): the 16 chunk loads (K0..K7 then V0..V7) run RING-1 ahead.
constexpr int kRing = 5;  // 5 slots x 8 KiB x 4 waves = the 160 KiB of a CU at d=128

// Per-lane offsets of the loads of one 32-key chunk (load n covers keys
// 32C + n*KPI.., the same offsets for every chunk C).
template <int D>
struct ChunkLaneOffs {
  static constexpr int LOADS = 32 * KV<D>::ROWB / 1024;
  uint32_t k[LOADS], v[LOADS];
  __device__ __forceinline__ void init() {
    constexpr int KPI = kWave / KV<D>::CPR;
#pragma unroll
    for (int n = 0; n < LOADS; ++n) {
      k[n] = dma_lane_off<D, true>(n * KPI);
      v[n] = dma_lane_off<D, false>(n * KPI);
    }
  }
};

template <int D>
struct RingSrc {
  static constexpr int RING = kRing;
  static constexpr int SLOT = 32 * KV<D>::ROWB;      // bytes per chunk
  static constexpr int LOADS = SLOT / 1024;          // 1 KiB loads per chunk
  static constexpr int AHEAD = RING - 1;             // chunks in flight
  static_assert(LOADS * (AHEAD - 1) <= 63, "vmcnt range");
  const uint16_t* kc;
  const uint16_t* vc;
  const uint8_t* ring;  // RING * SLOT bytes owned by this wave
  SplitPages sp;
  int nkv, g, key0, last;
  const ChunkLaneOffs<D>* offs;  // used when the whole split is written (no clamping)

  template <int IDX>
  __device__ __forceinline__ void issue() const {
    constexpr int C = IDX & 7;
    constexpr int KPI = kWave / KV<D>::CPR;
    const uint32_t dst = (uint32_t)(uintptr_t)(ring + (IDX % RING) * SLOT);
    if (key0 + kSplit - 1 <= last) {
      const uint16_t* pool_g = (IDX < 8 ? kc : vc) + (int64_t)g * 16 * D;
      const uint32_t page_elems = (uint32_t)nkv * 16 * D;
      const uint32_t ring0 = (uint32_t)(uintptr_t)ring;
      static_for<0, LOADS>([&](auto nc) {
        constexpr int n = decltype(nc)::value;
        lds_dma16_si<(IDX % RING) * SLOT + n * 1024>(
            page_block(pool_g, sp.pg[(32 * C + n * KPI) >> 4], page_elems),
            IDX < 8 ? offs->k[n] : offs->v[n], ring0);
      });
      return;
    }
#pragma unroll
    for (int n = 0; n < LOADS; ++n) {
      const int kfirst = 32 * C + n * KPI;
      dma_block<D, (IDX < 8)>(IDX < 8 ? kc : vc, sp.pg[(32 * C + n * KPI) >> 4], nkv, g, key0,
                              kfirst, last, dst + (uint32_t)n * 1024);
    }
  }
  template <int IDX>
  __device__ __forceinline__ void prologue_from() const {
    if constexpr (IDX < AHEAD) {
      issue<IDX>();
      prologue_from<IDX + 1>();
    }
  }
  __device__ __forceinline__ void prologue() const { prologue_from<0>(); }
  template <int IDX>
  __device__ __forceinline__ void step() const {
    // chunks younger than IDX in flight: min(AHEAD - 1, 15 - IDX)
    wait_vmcnt_le<LOADS * (15 - IDX < AHEAD - 1 ? 15 - IDX : AHEAD - 1)>();
    // slot (IDX + AHEAD) % RING held chunk IDX - 1: its reads must have
    // returned before the refill can land
    if constexpr (IDX + AHEAD < 16) {
      lds_reads_done();
      issue<IDX + AHEAD>();
    }
  }
  template <int C>
  __device__ __forceinline__ u32x4 k(int h, int t) const {
    return lds_k_operand<D>(ring + (C % RING) * SLOT, h, t);
  }
  template <int C>
  __device__ __forceinline__ bf16x8 v(int i) const {
    return lds_v_operand<D>(ring + ((8 + C) % RING) * SLOT, i);
  }
};

// Eight int16 values (a K or V operand of the int16 cache) as two exact bf16
// operands: hi = bf16(v) and lo = bf16(v - hi); v has at most 16 significant
// bits, so hi + lo == v exactly and an MFMA with hi then lo adds v * b.
__device__ __forceinline__ void unpack_i16x8(u32x4 raw, bf16x8& hi, bf16x8& lo) {
  u32x4 h, l;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a = (float)(int16_t)(raw[j] & 0xffffu);
    const float b = (float)(int16_t)(raw[j] >> 16);
    h[j] = pack_bf16x2(a, b);
    l[j] = pack_bf16x2(a - bf16_lo(h[j]), b - bf16_hi(h[j]));
  }
  hi = as_bf16x8(h);
  lo = as_bf16x8(l);
}

// ---- the split partial, in two phases -----------------------------------------
// Lane l (r = l%16, q = l/16) owns column r of each of its NB blocks; block b's
// query sits at position pcol[b]; key j is valid iff j <= pcol[b] and
// j < key_end.  split_qk computes the logits, then per block m (base-2 max
// logit, -inf if nothing valid) and l (sum of e = exp2(z - m) in fp32, 0 where
// invalid), and leaves in p[b][c] the bf16 weights of keys key0+32c+8q+0..7.
// pmin (wave-uniform) is at most the position of every column whose result is
// used: a chunk whose last key is <= pmin and < key_end needs no masking.
// LDS operand reads are issued this many MFMA operands ahead of their use, so
// their latency hides behind the MFMAs in between (one wave per SIMD: nothing
// else would hide it).
constexpr int kOperandsAhead = 6;

// Whether an operand source reads the int16 cache (Src::Q16, default false).
template <class S, class = void>
struct SrcQ16 : std::false_type {};
template <class S>
struct SrcQ16<S, std::void_t<decltype(S::Q16)>> : std::integral_constant<bool, S::Q16> {};

template <int D, int NB, class Src>
__device__ __forceinline__ void split_qk(const Src& src, int key0, int key_end, int pmin,
                                         const bf16x8 (&qf)[NB][KV<D>::DS], const int (&pcol)[NB],
                                         float c2, u32x4 (&p)[NB][8], float (&m)[NB],
                                         float (&l)[NB]) {
  constexpr int DS = KV<D>::DS;
  constexpr int OPC = 2 * DS;      // K operands per 32-key chunk: (half h, d-step t)
  constexpr int NOP = 8 * OPC;
  constexpr int PD = kOperandsAhead;
  constexpr bool Q16 = SrcQ16<Src>::value;
  const int q = (threadIdx.x & (kWave - 1)) >> 4;
  float z[NB][8][8];
  u32x4 buf[PD];
  // operand o = (chunk c, half h, d-step t); a chunk's first read waits for
  // (and lets the source refill around) that chunk
  auto read = [&](auto oc) __attribute__((always_inline)) {
    constexpr int o = decltype(oc)::value;
    constexpr int c = o / OPC, h = (o % OPC) / DS, t = o % DS;
    if constexpr (o % OPC == 0) src.template step<c>();
    buf[o % PD] = src.template k<c>(h, t);
  };
  static_for<0, PD>(read);
  f32x4 acc[NB][2];
  static_for<0, NOP>([&](auto oc) __attribute__((always_inline)) {
    constexpr int o = decltype(oc)::value;
    constexpr int c = o / OPC, h = (o % OPC) / DS, t = o % DS;
    if constexpr (o % OPC == 0) {
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[b][0] = acc[b][1] = f32x4{};
    }
    const u32x4 raw = buf[o % PD];
    if constexpr (o + PD < NOP) read(std::integral_constant<int, o + PD>{});
    if constexpr (Q16) {
      bf16x8 hi, lo;
      unpack_i16x8(raw, hi, lo);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        acc[b][h] = mfma16(hi, qf[b][t], acc[b][h]);
        acc[b][h] = mfma16(lo, qf[b][t], acc[b][h]);
      }
    } else {
      const bf16x8 a = as_bf16x8(raw);
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[b][h] = mfma16(a, qf[b][t], acc[b][h]);
    }
    if constexpr (o % OPC == OPC - 1) {
      // dot products (int16 cache: times the key's factor); -inf marks an
      // invalid key
      float fk[8];
      if constexpr (Q16) src.kscale(c, fk);
      auto dot = [&](int b, int hh, int i) __attribute__((always_inline)) {
        if constexpr (Q16) return acc[b][hh][i] * fk[4 * hh + i];
        else return acc[b][hh][i];
      };
      const int last = key0 + 32 * c + 31;
      if (last <= pmin && last < key_end) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int i = 0; i < 4; ++i) z[b][c][4 * hh + i] = dot(b, hh, i);
      } else {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = key0 + 32 * c + 8 * q + 4 * hh + i;
              const bool ok = key <= pcol[b] && key < key_end;
              z[b][c][4 * hh + i] = ok ? dot(b, hh, i) : -INFINITY;
            }
      }
    }
  });
  // max, exponentials, sum: fixed order (chunks, then keys, then lanes).
  // The base-2 logit of a key is s*c2 for its dot product s.  Rounding is
  // monotone, so the largest rounded logit is round(max s * c2): the max is
  // taken over the raw dot products and scaled once.  Each exponent is
  // exp2(s*c2 - m) with s*c2 - m rounded once (fma).
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float mm = -INFINITY;
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) mm = fmaxf(mm, z[b][c][j]);
    mm = fmaxf(mm, __shfl_xor(mm, 16));
    mm = fmaxf(mm, __shfl_xor(mm, 32));
    mm = mm * c2;
    // with no valid key every s is -inf; subtracting 0 keeps exp2(-inf) = 0
    const float ms = mm == -INFINITY ? 0.0f : mm;
    float ll = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        e[j] = fast_exp2(fmaf(z[b][c][j], c2, -ms));
        ll = ll + e[j];
      }
      if constexpr (Q16) {
        // the value factor goes into the weight (the sum l keeps e itself); an
        // invalid key has e = 0 and its factor may be anything
        float fv[8];
        src.vscale(c, fv);
#pragma unroll
        for (int j = 0; j < 8; ++j) e[j] = e[j] != 0.0f ? e[j] * fv[j] : 0.0f;
      }
      p[b][c] = u32x4{pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]), pack_bf16x2(e[4], e[5]),
                      pack_bf16x2(e[6], e[7])};
    }
    ll = ll + __shfl_xor(ll, 16);
    ll = ll + __shfl_xor(ll, 32);
    m[b] = mm;
    l[b] = ll;
  }
}

// O^T = V^T P^T over the split's chunks in ascending order; o[b][i][t] holds
// dim 16i+4q+t of this lane's column in block b.
template <int D, int NB, class Src>
__device__ __forceinline__ void split_pv(const Src& src, const u32x4 (&p)[NB][8],
                                         f32x4 (&o)[NB][KV<D>::DB]) {
  constexpr int DB = KV<D>::DB;
  constexpr int NOP = 8 * DB;      // V operands: (chunk c, dim block i)
  constexpr int PD = kOperandsAhead;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < DB; ++i) o[b][i] = f32x4{};
  bf16x8 buf[PD];
  auto read = [&](auto oc) __attribute__((always_inline)) {
    constexpr int op = decltype(oc)::value;
    constexpr int c = op / DB, i = op % DB;
    if constexpr (i == 0) src.template step<8 + c>();
    buf[op % PD] = src.template v<c>(i);
  };
  static_for<0, PD>(read);
  static_for<0, NOP>([&](auto oc) __attribute__((always_inline)) {
    constexpr int op = decltype(oc)::value;
    constexpr int c = op / DB, i = op % DB;
    const bf16x8 va = buf[op % PD];
    if constexpr (op + PD < NOP) read(std::integral_constant<int, op + PD>{});
    if constexpr (SrcQ16<Src>::value) {
      bf16x8 hi, lo;
      unpack_i16x8(__builtin_bit_cast(u32x4, va), hi, lo);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        o[b][i] = mfma16(hi, as_bf16x8(p[b][c]), o[b][i]);
        o[b][i] = mfma16(lo, as_bf16x8(p[b][c]), o[b][i]);
      }
    } else {
#pragma unroll
      for (int b = 0; b < NB; ++b) o[b][i] = mfma16(va, as_bf16x8(p[b][c]), o[b][i]);
    }
  });
}

// Q^T operand for d-step t: dims 32t + 8q .. +7 of this lane's query row.
template <int D>
__device__ __forceinline__ void load_q(const uint16_t* qrow, bool live, bf16x8 (&qf)[KV<D>::DS]) {
  const int q = (threadIdx.x & (kWave - 1)) >> 4;
#pragma unroll
  for (int t = 0; t < KV<D>::DS; ++t) {
    const u32x4 v = live ? *(const u32x4*)(qrow + 32 * t + 8 * q) : u32x4{0u, 0u, 0u, 0u};
    settle(v);  // the untracked LDS loads that follow must not be waited on for q
    qf[t] = as_bf16x8(v);
  }
}

// Write one block's partial record (o[D], m, l, pad) for a live column:
// exactly STORES vector stores per wave (a live column always exists), which
// the decode stream counts in its waits.
template <int D>
struct PartialRec {
  static constexpr int FLOATS = attn_rec_floats(D);
  static constexpr int STORES = KV<D>::DB + 1;
};
template <int D>
__device__ __forceinline__ void store_partial(float* rec, const f32x4 (&o)[KV<D>::DB], float m,
                                              float l) {
  constexpr int DB = KV<D>::DB;
  const int qq = (threadIdx.x & (kWave - 1)) >> 4;
#pragma unroll
  for (int i = 0; i < DB; ++i) *(f32x4*)(rec + 16 * i + 4 * qq) = o[i];
  if (qq == 0) *(f32x2_t*)(rec + D) = f32x2_t{m, l};
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

// Int16 cache: each (token, kv head) row x of K or V is stored as
// q = rint(x * (32767 / s)) (int16, ties to even) with s = max |x| over the
// row, and its dequantisation factor f = s / 32767 (fp32; 0 for an all-zero
// row) in a [pages, n_kv, 16] array.  One wave per (token, kv head): the max
// is exact and order-free.
template <int D>
__global__ __launch_bounds__(64) void kv_append_i16_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ kv_len,
    const int32_t* __restrict__ bt, int16_t* __restrict__ kc, int16_t* __restrict__ vc,
    float* __restrict__ ks, float* __restrict__ vs, int nkv, int max_pages) {
  constexpr int PER = D / kWave;  // elements per lane
  const int b = blockIdx.y;
  const int i = blockIdx.x / nkv, g = blockIdx.x % nkv;
  int tok0 = b, nb = 1;
  if (cu_q != nullptr) {
    tok0 = cu_q[b];
    nb = cu_q[b + 1] - tok0;
  }
  if (i >= nb) return;
  const int lane = threadIdx.x;
  const int pos = kv_len[b] - nb + i;
  const int64_t tok = tok0 + i;
  const int page = bt[(int64_t)b * max_pages + (pos >> 4)];
  const int slot = pos & 15;
  const int64_t src = (tok * nkv + g) * D + lane * PER;
  const int64_t row = (((int64_t)page * nkv + g) << 4) + slot;
#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    const uint16_t* x = (kv ? v_new : k_new) + src;
    float v[PER];
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      v[e] = bf16_to_f32(x[e]);
      s = fmaxf(s, fabsf(v[e]));
    }
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) s = fmaxf(s, __shfl_xor(s, d));
    const float inv = 32767.0f / s;
    int16_t* dst = (kv ? vc : kc) + row * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      float qv = s > 0.0f ? rintf(v[e] * inv) : 0.0f;
      qv = fminf(fmaxf(qv, -32767.0f), 32767.0f);
      dst[e] = (int16_t)qv;
    }
    if (lane == 0) (kv ? vs : ks)[row] = s / 32767.0f;
  }
}

// ---- decode ------------------------------------------------------------------
// Persistent: one workgroup per CU (fewer if there are fewer units) of
// kDecodeWaves waves.  A unit is one (kv head g, sequence b, split s); wave w
// of NW processes units w, w + NW, w + 2NW, ... of the list of existing units.
// Each wave streams its units' chunks through a private ring of kDecodeSlots
// LDS slots without a break: while a unit's last chunks are computed, the next
// unit's first chunks are already loading; the next unit's block-table pages
// are read, and its q is copied into LDS, one unit ahead.  Full splits load
// their keys/values with the non-temporal hint (each byte is read once per
// call).
// Workspace record per (b, q head, s): o[D], m, l, 2 pad floats (fp32).
constexpr int kDecodeWaves = 2, kDecodeSlots = 8;  // slots divide the 16 chunks of a split
// The int16 cache's unpacking makes its units VALU-bound rather than
// HBM-bound: three waves per CU with a 4-slot ring each (the LDS holds no
// more), so three SIMDs do that work.
constexpr int kDecodeWaves16 = 3, kDecodeSlots16 = 4;
constexpr int kMapSeqs = 256;  // batches up to this size get the balanced unit list

template <int D>
struct DecodeUnit {
  SplitPages sp;
  int g, b, s, key0, last;
};

template <int D, int RING_, bool Q16_ = false>
struct StreamSrc {
  static constexpr bool Q16 = Q16_;                  // int16 cache
  static constexpr int RING = RING_;
  static constexpr int SLOT = 32 * KV<D>::ROWB;      // bytes per chunk
  static constexpr int LOADS = SLOT / 1024;          // 1 KiB loads per chunk
  static constexpr int AHEAD = RING - 1;             // chunks in flight
  // bf16 cache: the call's new key and value rows are written by the wave
  // that reads them (append)
  static constexpr bool APPEND = !Q16_;
  // q copy of the next unit, then (int16 cache) its key and value factors or
  // (bf16 cache) its sequence's new key and value rows
  static constexpr int QLOADS = 16 * KV<D>::ROWB / 1024 + 2;
  static constexpr int STORES = PartialRec<D>::STORES;    // previous unit's record
  static_assert(16 % RING == 0, "slots repeat every split");
  static_assert(LOADS * (AHEAD - 1) + STORES + QLOADS <= 63, "vmcnt range");
  uint16_t* kc;  // written only by append (bf16 cache)
  uint16_t* vc;
  const uint8_t* ring;
  const ChunkLaneOffs<D>* offs;
  int nkv;
  DecodeUnit<D> cur, nxt;
  bool has_next;
  bool first;  // the wave's first unit: no record stores precede its chunks
  // int16 cache: LDS addresses of the current unit's 256 key / value factors
  uint32_t kscl = 0, vscl = 0;
  // bf16 cache: LDS address of the next unit's staged new rows (key row at
  // +0, value row at +1024)
  uint32_t nstage = 0;

  // A unit that holds its sequence's last position writes that position's
  // key and value rows (staged in LDS at `stage`) into the pool before any
  // chunk of the unit is requested.  Its wave is the only reader of those
  // rows in the call, and its later loads see the stores: a wave's memory
  // operations on one address take effect in program order, and lanes of
  // one wave share the same vector L1.  Positions past the last re-read the
  // last row (dma_block), so every row loaded has been written.  The page
  // of the last position is pg[15] for every split that holds it.
  __device__ __forceinline__ void append(const DecodeUnit<D>& un, uint32_t stage) const {
    if (un.last - un.key0 >= kSplit) return;  // wave-uniform
    constexpr int CPR = KV<D>::CPR;
    const int lane = threadIdx.x & (kWave - 1), j = lane % CPR;
    const bool isv = lane >= CPR;
    const u32x4 x = *(lds_u32x4*)(uintptr_t)(stage + (isv ? 1024u : 0u) + 16u * (uint32_t)j);
    if (lane < 2 * CPR) {
      uint16_t* pool = isv ? vc : kc;
      const int64_t row = (((int64_t)un.sp.pg[15] * nkv + un.g) << 4) + (un.last & 15);
      *(u32x4*)(pool + row * D + 8 * j) = x;
    }
  }
  __device__ __forceinline__ void factors(uint32_t base, int C, float (&f)[8]) const {
    const int q = (threadIdx.x & (kWave - 1)) >> 4;
    const uint32_t a = base + (uint32_t)(32 * C + 8 * q) * 4;
    const f32x4 x = *(lds_f32x4*)(uintptr_t)a, y = *(lds_f32x4*)(uintptr_t)(a + 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[j] = x[j];
      f[4 + j] = y[j];
    }
  }
  __device__ __forceinline__ void kscale(int C, float (&f)[8]) const { factors(kscl, C, f); }
  __device__ __forceinline__ void vscale(int C, float (&f)[8]) const { factors(vscl, C, f); }

  // stream position G: chunk G of the current unit (G < 16) or chunk G-16 of
  // the next one; K chunks are 0..7, V chunks 8..15
  template <int G>
  __device__ __forceinline__ void issue() const {
    constexpr int C = G % 16, CC = C & 7;
    constexpr bool IS_K = C < 8;
    constexpr int KPI = kWave / KV<D>::CPR;
    const DecodeUnit<D>& un = G < 16 ? cur : nxt;
    const uint32_t dst = (uint32_t)(uintptr_t)(ring + (G % RING) * SLOT);
    const uint16_t* pool = IS_K ? kc : vc;
    if (un.key0 + kSplit - 1 <= un.last) {
      const uint16_t* pool_g = pool + (int64_t)un.g * 16 * D;
      const uint32_t page_elems = (uint32_t)nkv * 16 * D;
      const uint32_t ring0 = (uint32_t)(uintptr_t)ring;
      static_for<0, LOADS>([&](auto nc) {
        constexpr int n = decltype(nc)::value;
        lds_dma16_si<(G % RING) * SLOT + n * 1024, true>(
            page_block(pool_g, un.sp.pg[(32 * CC + n * KPI) >> 4], page_elems),
            IS_K ? offs->k[n] : offs->v[n], ring0);
      });
      return;
    }
#pragma unroll
    for (int n = 0; n < LOADS; ++n)
      // the last split re-reads the last key for positions past the end:
      // no streaming hint here, so those repeats hit in cache
      dma_block<D, IS_K>(pool, un.sp.pg[(32 * CC + n * KPI) >> 4], nkv, un.g, un.key0,
                         32 * CC + n * KPI, un.last, dst + (uint32_t)n * 1024);
  }
  template <int G>
  __device__ __forceinline__ void prologue_from() const {
    if constexpr (G < AHEAD) {
      issue<G>();
      prologue_from<G + 1>();
    }
  }
  __device__ __forceinline__ void prologue() const { prologue_from<0>(); }
  // Before chunk IDX of the current unit is read: wait for it, then refill
  // the slot of chunk IDX-1.  The operations issued after chunk IDX are the
  // next AHEAD-1 stream chunks and, while IDX < AHEAD, the previous unit's
  // record stores (unless this is the wave's first unit) and the next unit's
  // q copy.  Without a next unit the wait counts only the chunks that follow,
  // and the next unit's append stores (ahead of its first chunk) are not
  // counted either (waiting for more is never wrong).
  template <int IDX>
  __device__ __forceinline__ void step() const {
    if (has_next) {
      if constexpr (IDX < AHEAD) {
        if (first) wait_vmcnt_le<LOADS * (AHEAD - 1) + QLOADS>();
        else wait_vmcnt_le<LOADS * (AHEAD - 1) + STORES + QLOADS>();
      } else {
        wait_vmcnt_le<LOADS * (AHEAD - 1)>();
      }
      lds_reads_done();
      // the next unit's first chunk: its append comes first (its staged rows
      // arrived with its q copy, which the waits so far have covered)
      if constexpr (APPEND && IDX + AHEAD == 16) append(nxt, nstage);
      issue<IDX + AHEAD>();
    } else {
      wait_vmcnt_le<LOADS * (15 - IDX < AHEAD - 1 ? 15 - IDX : AHEAD - 1)>();
      if constexpr (IDX + AHEAD < 16) {
        lds_reads_done();
        issue<IDX + AHEAD>();
      }
    }
  }
  template <int C>
  __device__ __forceinline__ u32x4 k(int h, int t) const {
    return lds_k_operand<D>(ring + (C % RING) * SLOT, h, t);
  }
  template <int C>
  __device__ __forceinline__ bf16x8 v(int i) const {
    return lds_v_operand<D>(ring + ((8 + C) % RING) * SLOT, i);
  }
};

// The q of a unit (16 columns = the group's heads, padded with copies of a
// live column, x D) in LDS: column rows of D*2 bytes with their 16-byte chunks
// XOR-swizzled by column so that the 16 columns a read covers fall on distinct
// banks.
template <int D>
__device__ __forceinline__ int qswz(int col) {
  if constexpr (D == 128) return col & 15;
  else return (col >> 1) & 7;
}
template <int D>
__device__ __forceinline__ void copy_q(const uint16_t* q, int b, int g, int nq, int group,
                                       uint32_t slot) {
  constexpr int CPR = KV<D>::CPR;
  const int lane = threadIdx.x & (kWave - 1);
  const uint16_t* base = q + ((int64_t)b * nq + (int64_t)g * group) * D;
#pragma unroll
  for (int n = 0; n < 16 * CPR / kWave; ++n) {
    const int idx = n * kWave + lane, col = idx / CPR, phys = idx % CPR;
    const int logical = phys ^ qswz<D>(col);
    const int src_col = min(col, group - 1);
    lds_dma16_sv(base, (uint32_t)((src_col * D + logical * 8) * 2), slot + (uint32_t)n * 1024);
  }
}
// Lane I of x takes the wave-uniform value v (v_writelane_b32; the lane
// select is an inline constant).
template <int I>
__device__ __forceinline__ void write_lane(int& x, int v) {
  asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(x) : "s"(v), "i"(I));
}

// The key and value factors of a decode unit's 256 keys (int16 cache) into
// LDS: lane l brings keys key0 + 4l .. +3, slots 4(l%4).. of page pg[l/4]
// (for a split past the last position the page is the last one's; those
// keys' factors are never used).  Two direct loads of 1 KiB.
template <int D>
__device__ __forceinline__ void copy_factors(const float* kf, const float* vf,
                                             const DecodeUnit<D>& un, int nkv, uint32_t slot) {
  const int lane = threadIdx.x & (kWave - 1);
  // lane i of `held` holds pg[i] (the pages are wave-uniform); lane l then
  // reads lane l/4's value.  (A select chain over pg here is turned into an
  // indexed access, which would put the whole unit in scratch memory.)
  int held = 0;
  static_for<0, 16>([&](auto ic) __attribute__((always_inline)) {
    write_lane<decltype(ic)::value>(held, un.sp.pg[decltype(ic)::value]);
  });
  const int page = __builtin_amdgcn_ds_bpermute((lane >> 2) << 2, held);
  const uint32_t off = (uint32_t)((((int64_t)page * nkv + un.g) * 16 + 4 * (lane & 3)) * 4);
  lds_dma16_sv(kf, off, slot);
  lds_dma16_sv(vf, off, slot + 1024);
}

// The new key and value rows of a unit's (sequence, kv head) -- the rows of
// its last position, in [sequence, kv head, D] arrays -- into LDS: the key row
// at slot, the value row at slot + 1024, 16-byte chunk j at +16j (the lanes
// past one row's chunks repeat them).  Two direct loads of 1 KiB.
template <int D>
__device__ __forceinline__ void copy_new_rows(const uint16_t* k_new, const uint16_t* v_new,
                                              const DecodeUnit<D>& un, int nkv, uint32_t slot) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = ((int64_t)un.b * nkv + un.g) * D;
  const uint32_t off = (uint32_t)(lane % KV<D>::CPR) * 16u;
  lds_dma16_sv(k_new + row, off, slot);
  lds_dma16_sv(v_new + row, off, slot + 1024);
}

template <int D>
__device__ __forceinline__ void read_q(const uint8_t* slot, bf16x8 (&qf)[KV<D>::DS]) {
  const int lane = threadIdx.x & (kWave - 1), col = lane & 15, q4 = lane >> 4;
#pragma unroll
  for (int t = 0; t < KV<D>::DS; ++t)
    qf[t] = as_bf16x8(*(const u32x4*)(slot + col * KV<D>::ROWB + (((4 * t + q4) ^ qswz<D>(col)) << 4)));
}

// Q16: the cache holds int16 codes with per-(page, kv head, slot) factors kf /
// vf; each unit's 256 key and value factors travel with its q copy into a
// double-buffered 2 KiB LDS slot of the wave.  Otherwise (bf16 cache) the
// kernel also appends the call's token: k_new / v_new hold each sequence's
// new key and value rows ([B, nkv, D]), which belong at position kv_len - 1;
// the same slots carry them (StreamSrc::append).
template <int D, int WAVES, int RING, bool Q16>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bi_attn_decode_partial_kernel(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ kv_len,
    const int32_t* __restrict__ bt, uint16_t* __restrict__ kc, uint16_t* __restrict__ vc,
    float* __restrict__ ws, int B, int nq, int nkv, int max_pages, int smax, float c2,
    const float* __restrict__ kf, const float* __restrict__ vf,
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new) {
  using Src = StreamSrc<D, RING, Q16>;
  constexpr int QSLOT = 16 * KV<D>::ROWB;
  // int16 cache: key factors, then value factors; bf16 cache: the new key
  // row, then the new value row (1 KiB each: one direct load apiece)
  constexpr int FSLOT = 2048;
  __shared__ __attribute__((aligned(1024)))
  uint8_t lds[WAVES][Src::RING * Src::SLOT + 2 * QSLOT + 2 * FSLOT];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t NW = (int64_t)gridDim.x * WAVES;
  const int64_t total = (int64_t)B * nkv * smax;
  const int group = nq / nkv;
  const uint8_t* ring = lds[wave];
  const uint32_t qslot0 = (uint32_t)(uintptr_t)(ring + Src::RING * Src::SLOT);
  const uint32_t fslot0 = qslot0 + 2 * QSLOT;

  // Units are dealt round-robin from the list of existing ones only, so every
  // wave gets the same number (+-1).  The list is sequence-major; sequence b
  // has nkv * ceil(L_b/256) units, kv head fastest.  For up to kMapSeqs
  // sequences, a per-lane prefix of those counts (64 sequences per register)
  // is built once and unit v is located by ballot; larger batches use the
  // dense (g, b, s) enumeration and skip splits past a sequence's end.
  constexpr int NCH = kMapSeqs / 64;
  int incl[NCH];  // inclusive prefix of per-sequence split counts, lane = sequence mod 64
  int64_t listed = 0;
  const bool mapped = B <= kMapSeqs;
  if (mapped) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int bi = c * 64 + lane;
      // at most smax splits whatever kv_len holds: a length past the call's
      // bound never addresses records beyond its sequence's
      const int ns = bi < B ? min(smax, (kv_len[bi] + kSplit - 1) / kSplit) : 0;
      int x = ns;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d);
        if (lane >= d) x += y;
      }
      incl[c] = x + (int)(listed / nkv);
      listed += (int64_t)__builtin_amdgcn_readlane(x, 63) * nkv;
    }
  }
  const int64_t total_units = mapped ? listed : total;
  // the first unit at or after u that exists (total_units if none)
  auto next_valid = [&](int64_t u) {
    if (mapped) return u < total_units ? u : total_units;
    for (; u < total; u += NW) {
      const int b = (int)((u / nkv) % B), s = (int)(u / nkv / B);
      if (s * kSplit < kv_len[b]) break;
    }
    return u;
  };
  auto fill = [&](DecodeUnit<D>& un, int64_t u) {
    if (mapped) {
      const int64_t sp = u / nkv;  // split index in the sequence-major list
      int b = 0;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        // sequences of this register whose splits all come before sp
        b += __builtin_popcountll(__ballot((int64_t)incl[c] <= sp));
      }
      // splits of the sequences before b: the inclusive prefix of sequence b-1
      int before = 0;
#pragma unroll
      for (int c = 0; c < NCH; ++c)
        if (b >= 1 && (b - 1) / 64 == c) before = __builtin_amdgcn_readlane(incl[c], (b - 1) % 64);
      un.b = b;
      un.s = (int)(sp - before);
      un.g = (int)(u % nkv);
    } else {
      un.g = (int)(u % nkv);
      un.b = (int)((u / nkv) % B);
      un.s = (int)(u / nkv / B);
    }
    // every field is wave-uniform; say so, so that they live in scalar registers
    un.g = __builtin_amdgcn_readfirstlane(un.g);
    un.b = __builtin_amdgcn_readfirstlane(un.b);
    un.s = __builtin_amdgcn_readfirstlane(un.s);
    un.key0 = un.s * kSplit;
    un.last = __builtin_amdgcn_readfirstlane(kv_len[un.b] - 1);
    un.sp.load(bt + (int64_t)un.b * max_pages, un.key0, un.last);
  };

  int64_t u = next_valid((int64_t)blockIdx.x * WAVES + wave);
  if (u >= total_units) return;
  ChunkLaneOffs<D> offs;
  offs.init();
  Src src{kc, vc, ring, &offs, nkv, {}, {}, false, true};
  fill(src.cur, u);
  int qi = 0;
  if constexpr (Src::APPEND) {
    // the wave's first unit: its append, when it has one, ahead of everything
    if (src.cur.last - src.cur.key0 < kSplit) {
      copy_new_rows<D>(k_new, v_new, src.cur, nkv, fslot0);
      wait_vmcnt_le<0>();
      src.append(src.cur, fslot0);
    }
  }
  copy_q<D>(q, src.cur.b, src.cur.g, nq, group, qslot0);
  if constexpr (Q16) copy_factors<D>(kf, vf, src.cur, nkv, fslot0);
  src.prologue();
  const int col = lane & 15;
  const bool live = col < group;
  while (true) {
    const int64_t un = next_valid(u + NW);
    src.has_next = un < total_units;
    if (src.has_next) {
      fill(src.nxt, un);
      copy_q<D>(q, src.nxt.b, src.nxt.g, nq, group, qslot0 + (uint32_t)(qi ^ 1) * QSLOT);
      if constexpr (Q16) {
        copy_factors<D>(kf, vf, src.nxt, nkv, fslot0 + (uint32_t)(qi ^ 1) * FSLOT);
      } else {
        // staged for every next unit, so that the wait counts stay fixed;
        // used only by one that holds its sequence's last position
        src.nstage = fslot0 + (uint32_t)(qi ^ 1) * FSLOT;
        copy_new_rows<D>(k_new, v_new, src.nxt, nkv, src.nstage);
      }
    }
    // Wait for this unit's q copy.  Issued after it: the unit's first AHEAD
    // chunks, the previous unit's record stores (unless this is the wave's
    // first unit) and the next unit's q copy (if there is a next unit).  The
    // count is capped at the counter's range: a smaller count only waits longer.
    constexpr int QA = Src::LOADS * Src::AHEAD;
    constexpr int QB = QA + Src::STORES;
    if (src.first) {
      if (src.has_next) wait_vmcnt_le<QA + Src::QLOADS>();
      else wait_vmcnt_le<QA>();
    } else {
      if (src.has_next) wait_vmcnt_le<(QB + Src::QLOADS < 63 ? QB + Src::QLOADS : 63)>();
      else wait_vmcnt_le<(QB < 63 ? QB : 63)>();
    }
    bf16x8 qf[1][KV<D>::DS];
    read_q<D>(ring + Src::RING * Src::SLOT + qi * QSLOT, qf[0]);
    if constexpr (Q16) {
      src.kscl = fslot0 + (uint32_t)qi * FSLOT;
      src.vscl = src.kscl + 1024;
    }
    const int L = src.cur.last + 1;
    const int pcol[1] = {L - 1};
    u32x4 p[1][8];
    float m[1], l[1];
    f32x4 o[1][KV<D>::DB];
    split_qk<D, 1>(src, src.cur.key0, INT_MAX, L - 1, qf, pcol, c2, p, m, l);
    split_pv<D, 1>(src, p, o);
    if (live) {
      const int hq = src.cur.g * group + col;
      store_partial<D>(ws + (((int64_t)src.cur.b * nq + hq) * smax + src.cur.s) * PartialRec<D>::FLOATS, o[0],
                       m[0], l[0]);
    }
    if (!src.has_next) break;
    u = un;
    src.cur = src.nxt;
    src.first = false;
    qi ^= 1;
  }
  wait_vmcnt_le<0>();  // no LDS write may outlive the workgroup
}

// Fold the splits of one (sequence, q head) left in ascending order.
// The left fold  m' = max(m, m_s), a = 2^(m - m'), b = 2^(m_s - m'),
// l = fma(l, a, l_s b), o = fma(o, a, o_s b)  splits into what depends on the
// running state only through the max and what carries values from step to
// step.  The running max after split s is the prefix max M_s of the split
// maxima (fmaxf is exact, so any grouping gives the same M_s), and each step's
// coefficients a_s = 2^(M_{s-1} - M_s), b_s = 2^(m_s - M_s) follow from it
// alone: they are computed for a whole chunk of D splits at once (thread t:
// split s0 + t; prefix max by a wave scan, then across waves).  What stays
// sequential is the fma chain of l and of each output dim (thread d owns dim
// d), over the same values in the same order as the fold step by step, so the
// bits are those of fold_coef / fold_apply applied in turn.  A chunk (CH <= D
// splits: 16 when every sequence fits in 17 splits, 32 when in 33, else D) has
// all its records requested before its chain starts.
template <int D, int CH>
__global__ __launch_bounds__(D) void bi_attn_combine_kernel(const float* __restrict__ ws,
                                                            const int32_t* __restrict__ kv_len,
                                                            uint16_t* __restrict__ out,
                                                            float* __restrict__ lse, int nq,
                                                            int smax, int split_len) {
  static_assert(CH <= D, "one split per thread in the scan");
  constexpr int F = PartialRec<D>::FLOATS, NW = D / kWave;
  __shared__ float sa[CH], sb[CH], sl[CH], wmax[NW], mlast;
  const int64_t bh = blockIdx.x;
  const int b = (int)(bh / nq);
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const int L = kv_len[b];
  const int ns = min(smax, (L + split_len - 1) / split_len);
  const float* rec = ws + bh * smax * F;
  float M = rec[D], l = rec[D + 1], o = rec[t];  // split 0 is the initial state
  for (int s0 = 1; s0 < ns; s0 += CH) {
    const int n = min(CH, ns - s0);  // splits s0 .. s0+n-1 in this chunk
    // every record value of the thread's dim in the chunk, requested at once
    // (past the chunk's end the last split stands in: no branch per load)
    float po[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) po[j] = rec[(int64_t)(s0 + min(j, n - 1)) * F + t];
    // thread t: split s0+t's max; prefix max over the chunk, carried in
    const float* rt = rec + (int64_t)(s0 + min(t, n - 1)) * F;
    const float ms = t < n ? rt[D] : -INFINITY;
    float pm = ms;
#pragma unroll
    for (int k = 1; k < kWave; k <<= 1) {
      const float y = __shfl_up(pm, k);
      if (lane >= k) pm = fmaxf(pm, y);
    }
    if (lane == kWave - 1) wmax[wave] = pm;
    __syncthreads();
    float before = M;  // the running max before this wave's first split
#pragma unroll
    for (int w = 0; w < NW; ++w)
      if (w < wave) before = fmaxf(before, wmax[w]);
    pm = fmaxf(pm, before);                  // M_{s0+t}
    float prev = __shfl_up(pm, 1);           // M_{s0+t-1}
    if (lane == 0) prev = before;
    if (t < n) {
      const FoldCoef f = fold_coef(prev, ms);
      sa[t] = f.a;
      sb[t] = f.b;
      sl[t] = rt[D + 1];
    }
    if (t == n - 1) mlast = pm;
    __syncthreads();
    // the chains, in split order; steps past the chunk's end keep the state
    // by a select, so the chunk is one block
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const FoldCoef f{sa[j], sb[j], 0.0f};
      const bool ok = j < n;
      o = ok ? fold_apply(o, po[j], f) : o;
      l = ok ? fold_apply(l, sl[j], f) : l;
    }
    M = mlast;
    __syncthreads();  // every read of this chunk's arrays is done
  }
  out[bh * D + t] = (uint16_t)f32_to_bf16(o / l);
  if (lse != nullptr && t == 0) lse[bh] = lse_of(M, l);
}

// ---- prefill -----------------------------------------------------------------
// Grid (query tiles, kv heads, sequences); WAVES waves per workgroup, each
// wave NB blocks of 16/group positions x group heads.  Tiles run latest-first.
// Each 256-key split is copied into LDS (K, then V, by direct global->LDS
// loads) and shared by the workgroup's waves: V(s) loads while K(s) is used,
// K(s+1) while V(s) is used.  The two splits' rows fill most of a CU's LDS, so
// one workgroup runs per CU.  A launch with enough queries uses 8 waves (two
// per SIMD, whose MFMAs and softmax arithmetic then overlap, and each staged
// split serves twice the queries); a small one uses 4 waves so that its few
// queries still spread over all CUs.  A block's arithmetic is the same in
// every shape (the same MFMAs in the same order on the same operands), so a
// query's output bits depend on neither.

// Copy the K or V rows of a whole 256-key split into LDS: thread t's load n
// fills the 1 KiB block n*4 + t/64 (one page is 16 keys = 4 KiB at d=128,
// 2 KiB at d=64, so every load stays within one page).
// Per-lane offsets of a wave's staging loads: load n of wave w covers keys
// (4n + w)*KPI.., so kfirst mod 32 takes at most two values (by (4n*KPI/16)
// mod 2).
template <int D>
struct StageLaneOffs {
  uint32_t k[2], v[2];
  __device__ __forceinline__ void init(int wave) {
    constexpr int KPI = kWave / KV<D>::CPR;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      k[h] = dma_lane_off<D, true>(16 * h + wave * KPI);
      v[h] = dma_lane_off<D, false>(16 * h + wave * KPI);
    }
  }
};

// The int16 cache's factors of a split's 256 keys (one 1 KiB load by one
// wave: lane l brings keys key0 + 4l .. +3, in page (key0 + 4l)/16, read from
// the block table; past the last position the page is the last one's, and
// those keys' factors are never used).
__device__ __forceinline__ void stage_factors(const float* fpool, const int32_t* bt_row, int key0,
                                              int last, int nkv, int g, uint8_t* lds) {
  const int lane = threadIdx.x & (kWave - 1);
  const int page = bt_row[min(key0 + 4 * lane, last) >> 4];
  lds_dma16(fpool + (((int64_t)page * nkv + g) << 4) + 4 * (lane & 3),
            (uint32_t)(uintptr_t)lds);
}

// With an int16 cache the K stage also brings the split's key factors (wave
// 0) and value factors (wave 1): both are read while the logits and weights
// are formed, before the value rows are waited for.
struct SplitFactors {
  const float* kf = nullptr;
  const float* vf = nullptr;
  uint8_t* klds = nullptr;
  uint8_t* vlds = nullptr;
  const int32_t* bt_row = nullptr;
};

// WAVES waves share the copy: load n of wave w brings keys (WAVES*n + w)*KPI
// .. +KPI-1, which lie in page (WAVES*n*KPI)/16 + (w*KPI)/16 of the split.
// stage_part issues loads N0 .. N0+CNT-1 of the wave's NLOAD.
template <int D, int WAVES>
struct StageGeom {
  static constexpr int KPI = kWave / KV<D>::CPR;       // keys per 1 KiB load
  static constexpr int NLOAD = 256 / KPI / WAVES;      // loads per thread
  static_assert((WAVES * KPI) % 16 == 0 && KPI <= 16, "a load stays inside one page");
};
template <int D, bool IS_K, int WAVES, int N0, int CNT>
__device__ __forceinline__ void stage_part(const uint16_t* pool, const SplitPages& sp, int nkv,
                                           int g, int key0, int last, uint32_t base,
                                           const StageLaneOffs<D>& offs) {
  constexpr int KPI = StageGeom<D, WAVES>::KPI;
  static_assert(N0 >= 0 && CNT >= 0 && N0 + CNT <= StageGeom<D, WAVES>::NLOAD, "load range");
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int poff = (wave * KPI) >> 4;           // pages the wave's first key is past
  auto page_of = [&](int pidx) __attribute__((always_inline)) {
    if constexpr (WAVES * KPI <= 32) {           // poff is 0 or 1
      return poff != 0 ? sp.pg[min(pidx + 1, 15)] : sp.pg[pidx];
    } else {                                     // poff is 0..3
      const int a = poff & 1 ? sp.pg[min(pidx + 1, 15)] : sp.pg[pidx];
      const int b = poff & 1 ? sp.pg[min(pidx + 3, 15)] : sp.pg[min(pidx + 2, 15)];
      return poff & 2 ? b : a;
    }
  };
  if (key0 + kSplit - 1 <= last) {
    const uint16_t* pool_g = pool + (int64_t)g * 16 * D;
    const uint32_t page_elems = (uint32_t)nkv * 16 * D;
    const uint32_t wbase = base + (uint32_t)(wave * KPI * KV<D>::ROWB);
    static_for<N0, N0 + CNT>([&](auto nc) {
      constexpr int n = decltype(nc)::value;
      constexpr int pidx = (n * WAVES * KPI) >> 4;
      constexpr int h = ((n * WAVES * KPI) >> 4) & 1;
      lds_dma16_si<n * WAVES * KPI * KV<D>::ROWB>(page_block(pool_g, page_of(pidx), page_elems),
                                                  IS_K ? offs.k[h] : offs.v[h], wbase);
    });
    return;
  }
#pragma unroll
  for (int n = N0; n < N0 + CNT; ++n) {
    const int pidx = (n * WAVES * KPI) >> 4;    // compile-time after unrolling
    const int kfirst = (n * WAVES + wave) * KPI;
    dma_block<D, IS_K>(pool, page_of(pidx), nkv, g, key0, kfirst, last,
                       base + (uint32_t)kfirst * KV<D>::ROWB);
  }
}

template <int D, bool IS_K, int WAVES>
__device__ __forceinline__ void stage_split(const uint16_t* pool, const SplitPages& sp, int nkv,
                                            int g, int key0, int last, uint8_t* lds,
                                            const StageLaneOffs<D>& offs,
                                            const SplitFactors& fac = SplitFactors{}) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (IS_K && fac.kf != nullptr) {
    // before the row loads: the block-table read is waited for here, with no
    // direct load of this stage in flight yet
    if (wave == 0) stage_factors(fac.kf, fac.bt_row, key0, last, nkv, g, fac.klds);
    if (wave == 1) stage_factors(fac.vf, fac.bt_row, key0, last, nkv, g, fac.vlds);
  }
  stage_part<D, IS_K, WAVES, 0, StageGeom<D, WAVES>::NLOAD>(pool, sp, nkv, g, key0, last,
                                                          (uint32_t)(uintptr_t)lds, offs);
}

// The bf16 prefill source with the stage loads spread over the chunks: the
// value rows of split s are issued over the first STEPS 32-key chunks of its
// logits, the key rows of split s+1 over the first STEPS chunks of its
// weighted sum (which start once every wave is past the barrier that frees
// the buffer), so that the memory pipe works beside the MFMAs instead of
// holding every wave at one burst of loads.  Issuing them all at the first
// chunk, or spreading them over four or eight, measured slower than two.
template <int D, int WAVES, int STEPS>
struct SpreadSrc : StagedSrc<D> {
  static constexpr int NLOAD = StageGeom<D, WAVES>::NLOAD;
  static constexpr int NSTEP = STEPS < NLOAD ? STEPS : NLOAD;
  static constexpr int PER = NLOAD / NSTEP;
  static_assert(PER * NSTEP == NLOAD, "loads per step");
  const uint16_t* kc;
  const uint16_t* vc;
  SplitPages vpages, kpages;
  int nkv, g, vkey0, kkey0, last;
  bool kon;
  uint32_t klds, vlds;
  const StageLaneOffs<D>* offs;
  template <int IDX>
  __device__ __forceinline__ void step() const {
    constexpr int c = IDX % 8;
    if constexpr (c < NSTEP) {
      if constexpr (IDX < 8)
        stage_part<D, false, WAVES, c * PER, PER>(vc, vpages, nkv, g, vkey0, last, vlds, *offs);
      else if (kon)
        stage_part<D, true, WAVES, c * PER, PER>(kc, kpages, nkv, g, kkey0, last, klds, *offs);
    }
  }
};

// Q16: the cache holds int16 rows with per-(page, kv head, slot) factors
// kf / vf (nullptr otherwise).  cu_q == nullptr means one token per sequence.
template <int D, bool Q16, int NB, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void bi_attn_prefill_kernel(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ kv_len, const int32_t* __restrict__ bt,
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc, uint16_t* __restrict__ out,
    float* __restrict__ lse, int nq, int nkv, int max_pages, float c2,
    const float* __restrict__ kf, const float* __restrict__ vf) {
  constexpr int DB = KV<D>::DB;
  __shared__ __attribute__((aligned(1024))) uint8_t klds[256 * KV<D>::ROWB];
  __shared__ __attribute__((aligned(1024))) uint8_t vlds[256 * KV<D>::ROWB];
  __shared__ __attribute__((aligned(1024))) uint8_t flds[Q16 ? 2 * 1024 : 16];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // the workgroups of one (sequence, kv head) go to one XCD, whose L2 then
  // serves each split's rows to all of them; tiles in descending order, so
  // that the longest start first
  const uint32_t nwg = gridDim.x * gridDim.y * gridDim.z;
  const uint32_t lid =
      xcd_contiguous_id(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z), nwg);
  const uint32_t lrest = lid / gridDim.x;
  const int b = (int)(lrest / gridDim.y), g = (int)(lrest % gridDim.y);
  const int tile = (int)(gridDim.x - 1 - lid % gridDim.x);
  const int group = nq / nkv;
  const int ppb = 16 / group;  // positions per block
  const int per_wg = WAVES * NB * ppb;
  const int tok0 = cu_q != nullptr ? cu_q[b] : b;
  const int nb = cu_q != nullptr ? cu_q[b + 1] - tok0 : 1;
  if (tile * per_wg >= nb) return;  // whole workgroup: no barrier reached
  const int L = kv_len[b];
  const int start = L - nb;
  const int col = lane & 15;
  const int hq = g * group + col % group;
  bf16x8 qf[NB][KV<D>::DS];
  int pcol[NB];
  int64_t tok[NB];
  bool live[NB];
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    const int pi = tile * per_wg + (wave * NB + bb) * ppb + col / group;
    live[bb] = pi < nb;
    tok[bb] = tok0 + min(pi, nb - 1);
    load_q<D>(q + (tok[bb] * nq + hq) * D, live[bb], qf[bb]);
    pcol[bb] = live[bb] ? start + pi : -1;
  }
  const int pmax = start + min((tile + 1) * per_wg, nb) - 1;
  // the wave's columns are consecutive positions from its first one on; lanes
  // past the chunk's end are never stored or folded
  const int pmin = start + tile * per_wg + wave * NB * ppb;
  const int nsplit = pmax / kSplit + 1;
  const int32_t* bt_row = bt + (int64_t)b * max_pages;
  constexpr int kSpreadSteps = 2;
  using Src = std::conditional_t<Q16, StagedSrc16<D>, SpreadSrc<D, WAVES, kSpreadSteps>>;
  Src src;
  src.ol.init((uint32_t)(uintptr_t)klds, (uint32_t)(uintptr_t)vlds);
  SplitFactors fac;
  if constexpr (Q16) {
    fac = SplitFactors{kf, vf, flds, flds + 1024, bt_row};
    src.kscl = (uint32_t)(uintptr_t)fac.klds;
    src.vscl = (uint32_t)(uintptr_t)fac.vlds;
  }

  float M[NB], Lsum[NB];
  f32x4 O[NB][DB];
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    M[bb] = -INFINITY;
    Lsum[bb] = 0.0f;
#pragma unroll
    for (int i = 0; i < DB; ++i) O[bb][i] = f32x4{};
  }
  SplitPages pages;
  pages.load(bt_row, 0, L - 1);
  StageLaneOffs<D> soffs;
  soffs.init(wave);
  stage_split<D, true, WAVES>(kc, pages, nkv, g, 0, L - 1, klds, soffs, fac);
  if constexpr (!Q16) {
    src.kc = kc;
    src.vc = vc;
    src.nkv = nkv;
    src.g = g;
    src.last = L - 1;
    src.klds = (uint32_t)(uintptr_t)klds;
    src.vlds = (uint32_t)(uintptr_t)vlds;
    src.offs = &soffs;
  }
  for (int s = 0; s < nsplit; ++s) {
    const int key0 = s * kSplit;
    wait_vmcnt_le<0>();
    __syncthreads();  // K(s) in LDS; every wave is done reading V(s-1)
    if constexpr (Q16) stage_split<D, false, WAVES>(vc, pages, nkv, g, key0, L - 1, vlds, soffs);
    SplitPages next;  // the next split's pages, fetched while this one computes
    if (s + 1 < nsplit) next.load(bt_row, key0 + kSplit, L - 1);
    if constexpr (!Q16) {
      src.vpages = pages;
      src.vkey0 = key0;
      src.kpages = next;
      src.kkey0 = key0 + kSplit;
      src.kon = s + 1 < nsplit;
    }
    u32x4 p[NB][8];
    float ms[NB], ls[NB];
    split_qk<D, NB>(src, key0, INT_MAX, pmin, qf, pcol, c2, p, ms, ls);
    wait_vmcnt_le<0>();
    __syncthreads();  // V(s) in LDS; every wave is done reading K(s)
    if (s + 1 < nsplit) {
      pages = next;
      if constexpr (Q16)
        stage_split<D, true, WAVES>(kc, pages, nkv, g, key0 + kSplit, L - 1, klds, soffs, fac);
    }
    f32x4 os[NB][DB];
    split_pv<D, NB>(src, p, os);
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      if (key0 <= pcol[bb]) {
        if (s == 0) {
          M[bb] = ms[bb];
          Lsum[bb] = ls[bb];
#pragma unroll
          for (int i = 0; i < DB; ++i) O[bb][i] = os[bb][i];
        } else {
          const FoldCoef f = fold_coef(M[bb], ms[bb]);
          Lsum[bb] = fold_apply(Lsum[bb], ls[bb], f);
#pragma unroll
          for (int i = 0; i < DB; ++i)
#pragma unroll
            for (int t = 0; t < 4; ++t) O[bb][i][t] = fold_apply(O[bb][i][t], os[bb][i][t], f);
          M[bb] = f.m;
        }
      }
    }
  }
  const int qq = lane >> 4;
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    if (!live[bb]) continue;
    const int64_t orow = (tok[bb] * nq + hq) * D;
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        out[orow + 16 * i + 4 * qq + t] = (uint16_t)f32_to_bf16(O[bb][i][t] / Lsum[bb]);
    if (lse != nullptr && qq == 0) lse[tok[bb] * nq + hq] = lse_of(M[bb], Lsum[bb]);
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
  __shared__ __attribute__((aligned(1024))) uint8_t ring[4][kRing * RingSrc<D>::SLOT];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t u = (int64_t)blockIdx.x * 4 + wave;
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
  bf16x8 qf[1][KV<D>::DS];
  load_q<D>(q + ((int64_t)b * nq + hq) * D, live, qf[0]);
  const int pcol[1] = {L - 1};
  float M = -INFINITY, Lsum = 0.0f;
  f32x4 O[DB];
  ChunkLaneOffs<D> offs;
  offs.init();
  for (int key0 = k_begin; key0 < k_end; key0 += kSplit) {
    RingSrc<D> src{kc, vc, ring[wave], {}, nkv, g, key0, L - 1, &offs};
    src.sp.load(bt + (int64_t)b * max_pages, key0, L - 1);
    src.prologue();
    u32x4 p[1][8];
    float ms[1], ls[1];
    f32x4 os[1][DB];
    split_qk<D, 1>(src, key0, k_end, L - 1, qf, pcol, c2, p, ms, ls);
    split_pv<D, 1>(src, p, os);
    if (key0 == k_begin) {
      M = ms[0];
      Lsum = ls[0];
#pragma unroll
      for (int i = 0; i < DB; ++i) O[i] = os[0][i];
    } else {
      const FoldCoef f = fold_coef(M, ms[0]);
      Lsum = fold_apply(Lsum, ls[0], f);
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int t = 0; t < 4; ++t) O[i][t] = fold_apply(O[i][t], os[0][i][t], f);
      M = f.m;
    }
  }
  if (live) store_partial<D>(ws + (((int64_t)b * nq + hq) * nsplit + sp) * PartialRec<D>::FLOATS, O,
                            M, Lsum);
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

// The wide prefill workgroup: NB blocks per wave x WAVES waves (NB * WAVES = 8).
constexpr int kWideNB = 1, kWideWaves = 8;

hipError_t launch_attn_prefill(const AttnDims& s, const void* q, const int32_t* cu_q,
                               const int32_t* kv_len, const int32_t* bt, const void* kc,
                               const void* vc, void* out, float* lse, int max_q_per_seq,
                               hipStream_t st, const float* kf, const float* vf) {
  const bool q16 = kf != nullptr;
  // A wide workgroup (8 waves of one block, or 4 waves of two) covers 32
  // positions; it is used (bf16 cache) when that still gives >= 4 workgroups
  // per CU: with fewer, the causal triangle's longest tiles decide the time and
  // the coarser split of the work costs what the wider tile saves.
  const int ppb = 16 / (s.nq / s.nkv);
  const int64_t wide_wgs = (int64_t)((max_q_per_seq + 8 * ppb - 1) / (8 * ppb)) * s.nkv * s.B;
  const bool wide = !q16 && wide_wgs >= 4 * (int64_t)device_cus();
  const int per_wg = (wide ? 8 : 4) * ppb;
  const dim3 grid((unsigned)((max_q_per_seq + per_wg - 1) / per_wg), (unsigned)s.nkv,
                  (unsigned)s.B);
  const float c2 = base2_scale(s.scale);
#define BI_PREFILL(DD, QQ, NN, WW)                                                             \
  hipLaunchKernelGGL((bi_attn_prefill_kernel<DD, QQ, NN, WW>), grid, dim3(64 * WW), 0, st,     \
                     (const uint16_t*)q, cu_q, kv_len, bt, (const uint16_t*)kc,                \
                     (const uint16_t*)vc, (uint16_t*)out, lse, s.nq, s.nkv, s.max_pages, c2, kf, \
                     vf)
  if (s.d == 128) {
    if (q16)
      BI_PREFILL(128, true, 1, 4);
    else if (wide)
      BI_PREFILL(128, false, kWideNB, kWideWaves);
    else
      BI_PREFILL(128, false, 1, 4);
  } else {
    if (q16)
      BI_PREFILL(64, true, 1, 4);
    else if (wide)
      BI_PREFILL(64, false, kWideNB, kWideWaves);
    else
      BI_PREFILL(64, false, 1, 4);
  }
#undef BI_PREFILL
  return hipGetLastError();
}

hipError_t launch_kv_append_i16(const AttnDims& s, const void* k_new, const void* v_new,
                                const int32_t* cu_q, const int32_t* kv_len, const int32_t* bt,
                                void* kc, void* vc, float* kf, float* vf, int max_q_per_seq,
                                hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)max_q_per_seq * s.nkv), (unsigned)s.B);
  if (s.d == 128)
    hipLaunchKernelGGL(kv_append_i16_kernel<128>, grid, dim3(64), 0, st, (const uint16_t*)k_new,
                       (const uint16_t*)v_new, cu_q, kv_len, bt, (int16_t*)kc, (int16_t*)vc, kf,
                       vf, s.nkv, s.max_pages);
  else
    hipLaunchKernelGGL(kv_append_i16_kernel<64>, grid, dim3(64), 0, st, (const uint16_t*)k_new,
                       (const uint16_t*)v_new, cu_q, kv_len, bt, (int16_t*)kc, (int16_t*)vc, kf,
                       vf, s.nkv, s.max_pages);
  return hipGetLastError();
}

// Workgroups of the persistent decode kernel: one per CU (each uses most of
// a CU's LDS), fewer when there are fewer units.
static int decode_workgroups(int64_t units, int waves) {
  const int cus = device_cus();
  const int64_t need = (units + waves - 1) / waves;
  return (int)(need < cus ? need : cus);
}

hipError_t launch_attn_decode(const AttnDims& s, const void* q, const void* k_new,
                              const void* v_new, const int32_t* kv_len, const int32_t* bt,
                              void* kc, void* vc, void* out, float* lse, int max_splits, float* ws,
                              hipStream_t st, const float* kf, const float* vf) {
  const int64_t units = (int64_t)s.B * s.nkv * max_splits;
  const bool q16 = kf != nullptr;
  const int waves = q16 ? kDecodeWaves16 : kDecodeWaves;
  const dim3 grid1((unsigned)decode_workgroups(units, waves)),
      grid2((unsigned)((int64_t)s.B * s.nq));
  const float c2 = base2_scale(s.scale);
#define BI_DECODE(DD, QQ)                                                                        \
  hipLaunchKernelGGL((bi_attn_decode_partial_kernel<DD, QQ ? kDecodeWaves16 : kDecodeWaves,      \
                                                    QQ ? kDecodeSlots16 : kDecodeSlots, QQ>),    \
                     grid1, dim3(64 * waves), 0, st, (const uint16_t*)q, kv_len, bt,             \
                     (uint16_t*)kc, (uint16_t*)vc, ws, s.B, s.nq, s.nkv, s.max_pages,           \
                     max_splits, c2, kf, vf, (const uint16_t*)k_new, (const uint16_t*)v_new)
  if (s.d == 128) {
    if (q16)
      BI_DECODE(128, true);
    else
      BI_DECODE(128, false);
    if (max_splits <= 17)
      hipLaunchKernelGGL((bi_attn_combine_kernel<128, 16>), grid2, dim3(128), 0, st,
                         (const float*)ws, kv_len, (uint16_t*)out, lse, s.nq, max_splits, kSplit);
    else if (max_splits <= 33)
      hipLaunchKernelGGL((bi_attn_combine_kernel<128, 32>), grid2, dim3(128), 0, st,
                         (const float*)ws, kv_len, (uint16_t*)out, lse, s.nq, max_splits, kSplit);
    else
      hipLaunchKernelGGL((bi_attn_combine_kernel<128, 128>), grid2, dim3(128), 0, st,
                         (const float*)ws, kv_len, (uint16_t*)out, lse, s.nq, max_splits, kSplit);
  } else {
    if (q16)
      BI_DECODE(64, true);
    else
      BI_DECODE(64, false);
    if (max_splits <= 17)
      hipLaunchKernelGGL((bi_attn_combine_kernel<64, 16>), grid2, dim3(64), 0, st,
                         (const float*)ws, kv_len, (uint16_t*)out, lse, s.nq, max_splits, kSplit);
    else if (max_splits <= 33)
      hipLaunchKernelGGL((bi_attn_combine_kernel<64, 32>), grid2, dim3(64), 0, st,
                         (const float*)ws, kv_len, (uint16_t*)out, lse, s.nq, max_splits, kSplit);
    else
      hipLaunchKernelGGL((bi_attn_combine_kernel<64, 64>), grid2, dim3(64), 0, st,
                         (const float*)ws, kv_len, (uint16_t*)out, lse, s.nq, max_splits, kSplit);
  }
#undef BI_DECODE
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
    hipLaunchKernelGGL((bi_attn_combine_kernel<128, 128>), grid2, dim3(128), 0, st,
                       (const float*)ws, kv_len, (uint16_t*)out, lse, s.nq, nsplit, split_len);
  } else {
    hipLaunchKernelGGL(bix_attn_decode_splitkv_kernel<64>, grid1, dim3(256), 0, st,
                       (const uint16_t*)q, kv_len, bt, (const uint16_t*)kc, (const uint16_t*)vc,
                       ws, s.B, s.nq, s.nkv, s.max_pages, nsplit, split_len, c2);
    hipLaunchKernelGGL((bi_attn_combine_kernel<64, 64>), grid2, dim3(64), 0, st,
                       (const float*)ws, kv_len, (uint16_t*)out, lse, s.nq, nsplit, split_len);
  }
  return hipGetLastError();
}

}  // namespace bi
