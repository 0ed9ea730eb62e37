// Device helpers shared by the libbi kernels (gfx950, wave64).
//
// Numerics policy for every kernel of the library: built with
// -ffp-contract=off and without fast-math, so a*b+c is always a rounded
// multiply followed by a rounded add unless a kernel asks for fmaf.  bf16
// results are rounded to nearest even by pack_bf16x2 / f32_to_bf16 below, the
// one conversion used everywhere.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace bi {

// Calls f(integral_constant<int, i>) for i = I .. N-1.
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Two floats -> two bf16 (lo in bits 0..15), round to nearest even; a NaN
// becomes the quiet NaN with the same sign and top payload bits
// ((bits >> 16) | 0x40); denormals are rounded, not flushed.  gfx950's
// v_cvt_pk_bf16_f32 implements exactly this rule (checked against the
// integer formulation over every upper half with boundary lower halves and
// 4M random patterns), two values per instruction.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.0f) & 0xffffu; }

// Low halves / high halves of two packed bf16 pairs: (lo16(a), lo16(b)) etc.
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// D(32x32) += A(32x16) * B(16x32), bf16 in, fp32 accumulate.
// Lane l: A row l%32, k = 8*(l/32)+0..7; B col l%32, same k;
// D col l%32, rows 8*(r/4) + 4*(l/32) + r%4 for register r.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D(16x16) += A(16x32) * B(32x16), bf16 in, fp32 accumulate.
// Lane l: A row l%16, k = 8*(l/16)+0..7; B col l%16, same k;
// D col l%16, rows 4*(l/16) + r for register r.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Direct global -> LDS load of 16 bytes per lane: lane l's bytes land at LDS
// address lds_base + 16*l (lds_base must be the same for the whole wave).  It
// is written as inline asm so that the compiler does not track it: its own
// conservative LDS-DMA tracking would wait for every load in flight before
// each LDS read and serialise the pipeline.  The kernel instead waits on the
// vector-memory counter explicitly (wait_vmcnt_le).  The instruction writes
// no VGPR, so there is no register the compiler could reuse while it runs.
// An LDS DMA that reads M0 must come at least one wait state after the SALU
// write of M0 (the compiler's hazard recognizer cannot see inside the asm, so
// the s_nop is written out here); without it the load may take the previous
// M0 and land in another LDS block.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is reserved; no compiler code here reads it
__device__ __forceinline__ void lds_dma16(const void* gptr, uint32_t lds_base) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(m0v), "v"(gptr)
               : "memory", "m0");
}
// The same load with a wave-uniform 64-bit base (scalar registers) plus a
// 32-bit per-lane byte offset, so a lane's address costs one register.
// STREAM sets the non-temporal hint: for data read once per call (the decode
// key/value stream), so that it does not displace lines the caches keep for
// reuse; data that is re-read (prefill, matmul operands) leaves it off.
template <bool STREAM = false>
__device__ __forceinline__ void lds_dma16_sv(const void* sbase, uint32_t voff, uint32_t lds_base) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_base);
  const uint64_t b = (uint64_t)(uintptr_t)sbase;
  // readfirstlane returns int: widen through uint32_t, never sign-extend
  const uint64_t ub =
      ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
      (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  if constexpr (STREAM)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                 :
                 : "s"(m0v), "v"(voff), "s"(ub)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(m0v), "v"(voff), "s"(ub)
                 : "memory", "m0");
}
// The same load to LDS address m0base + IMM (m0base wave-uniform): M0 is
// formed by one scalar add inside the asm.
template <int IMM, bool STREAM = false>
__device__ __forceinline__ void lds_dma16_si(const void* sbase, uint32_t voff, uint32_t m0base) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(m0base);
  const uint64_t b = (uint64_t)(uintptr_t)sbase;
  const uint64_t ub =
      ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
      (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  if constexpr (STREAM)
    asm volatile("s_add_u32 m0, %0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                 :
                 : "s"(m), "v"(voff), "s"(ub), "n"(IMM)
                 : "memory", "m0", "scc");
  else
    asm volatile("s_add_u32 m0, %0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(m), "v"(voff), "s"(ub), "n"(IMM)
                 : "memory", "m0", "scc");
}
#pragma clang diagnostic pop
// Make the compiler wait for a value's load here (an empty asm that reads
// it), before any untracked load is issued after it.
template <class T>
__device__ __forceinline__ void settle(const T& x) {
  asm volatile("" : : "v"(x));
}
// Wait until every LDS read this wave has issued has returned.  A direct
// global->LDS load writes LDS when its data arrives, with no ordering against
// LDS reads still queued ahead of it, so a buffer may be refilled only after
// this (or a workgroup barrier, whose fence waits the same way).  The memory
// clobber keeps the compiler from moving LDS reads across it.
__device__ __forceinline__ void lds_reads_done() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
// Two 4 x 16-bit transposed-read results as one 8 x bf16 MFMA operand
// (element 0 of `a` in bits 0..15 of the first dword).
__device__ __forceinline__ bf16x8 join_tr(s16x4 a, s16x4 b) {
  const u32x2 x = __builtin_bit_cast(u32x2, a), y = __builtin_bit_cast(u32x2, b);
  return as_bf16x8(u32x4{x[0], x[1], y[0], y[1]});
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (s_waitcnt with expcnt and lgkmcnt at their maxima, so only vmcnt waits).
template <int N>
__device__ __forceinline__ void wait_vmcnt_le() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroups are dispatched round-robin over the 8 XCDs (XCD = id % 8).
// Renumber so that each XCD receives one contiguous range of logical ids,
// which keeps neighbouring tiles in one XCD's L2.  A bijection for any count.
__device__ __forceinline__ uint32_t xcd_contiguous_id(uint32_t bid, uint32_t nwg) {
  const uint32_t q = nwg / 8u, r = nwg % 8u;
  const uint32_t xcd = bid % 8u, local = bid / 8u;
  return xcd * q + (xcd < r ? xcd : r) + local;
}

}  // namespace bi
