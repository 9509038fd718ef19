// Shared device helpers for the gfx950 MLA kernels: vector types, bf16 and
// e4m3fn conversions, LDS primitives, and the swizzled LDS layout of a cache page.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla.h"

#define MLA_LDS __attribute__((address_space(3)))

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef int v2i32_t __attribute__((ext_vector_type(2)));

namespace mla {

constexpr int kLatent = 512;
constexpr int kRope = 64;
constexpr int kRow = 576;
constexpr int kPage = 64;
constexpr int kRowBytesBf16 = 1152;
constexpr int kRowBytesFp8 = 584;
constexpr int kChunksPerRow = 72;                     // 16-byte chunks in a bf16 row
constexpr int kPageBytesBf16 = kPage * kRowBytesBf16; // 73728
constexpr int kPageBytesFp8 = kPage * kRowBytesFp8;   // 37376
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Wave / workgroup primitives
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// Workgroup barrier without a memory fence: waits for this wave's LDS ops, then
// s_barrier.  Global->LDS DMA completion is handled separately with vmcnt.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// v_permlane32_swap / v_permlane16_swap exchange halves (rows) of a wave in the VALU,
// without the LDS path a bpermute takes.  Called with the same register twice, the two
// results are this lane's value and that of lane ^ 32 (resp. ^ 16) in some order, so a
// commutative combine of the pair is the butterfly step.
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------------------
// LDS access with explicit address space
// ---------------------------------------------------------------------------
__device__ __forceinline__ bf16x8_t lds_read_b128(const MLA_LDS char* base, uint32_t byte_off) {
  return *reinterpret_cast<const MLA_LDS bf16x8_t*>(base + byte_off);
}

__device__ __forceinline__ bf16x4_t lds_read_tr16(const MLA_LDS char* base, uint32_t byte_off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      reinterpret_cast<MLA_LDS bf16x4_t*>(const_cast<MLA_LDS char*>(base) + byte_off));
}

// LDS reads at a 32-bit LDS byte address (a base the caller made opaque, plus a
// compile-time offset that lands in the instruction's offset field).
__device__ __forceinline__ bf16x8_t lds_read_b128_at(uint32_t addr) {
  return *reinterpret_cast<const MLA_LDS bf16x8_t*>((uintptr_t)addr);
}

__device__ __forceinline__ bf16x4_t lds_read_tr16_at(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(reinterpret_cast<MLA_LDS bf16x4_t*>((uintptr_t)addr));
}

// Hides a value from the optimiser: address arithmetic done on the result is not
// hoisted out of loops (where it would hold one register per unrolled access).
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// One 1 KiB global->LDS copy: lane l's 16 bytes at sbase + voff + IMM land at LDS
// byte address lds_base + LDS_ADD + 16 * l.  sbase must be wave-uniform (SGPR pair),
// voff a 32-bit per-lane offset, IMM < 4096.  The instruction adds its immediate to
// the LDS address as well as to the global one, so M0 gets LDS_ADD - IMM.
// Written as inline asm on purpose: the compiler does not see the LDS write, so it
// inserts no vmcnt(0) drain in front of later LDS reads of other buffers (it cannot
// prove they do not alias) and keeps no per-copy constants live.  Completion is the
// caller's business: each call is one vector-memory instruction for vmcnt.  M0 is
// set inside the statement; nothing else in these kernels keeps a value in M0.
template <int IMM, int LDS_ADD>
__device__ __forceinline__ void dma_16B(const void* sbase, uint32_t voff, uint32_t lds_base) {
  static_assert(IMM >= 0 && IMM < 4096, "immediate offset range");
  asm volatile(
      "s_add_u32 m0, %2, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1 offset:%4"
      :
      : "v"(voff), "s"(sbase), "s"(lds_base), "i"(LDS_ADD - IMM), "i"(IMM)
      : "memory", "scc");
}

__device__ __forceinline__ uint32_t lds_addr(const MLA_LDS void* p) {
  return (uint32_t)(uintptr_t)p;
}

// ---------------------------------------------------------------------------
// Layout of cache rows in LDS.  A block of 32 token rows x 72 chunks of 16 B (8 bf16)
// is stored column-group major: group G = c >> 3 (128 B of every row) holds the 32
// tokens x 8 chunks, and inside a group
// chunk c of token t sits at position t*8 + ((c & 7) ^ s(t)), byte 16 * slot, with
// s(t) = (t2, t1, t1 ^ t2 ^ t3) (bits 0, 1, 2 of s; ti = bit i of t).  gfx950 LDS has
// 64 banks of 4 bytes, so a 16-byte slot's bank group is slot & 15 = 8*(t & 1) + its
// position: same-parity tokens share one half of the banks.  Which lanes of an access
// are served together was read off SQ_LDS_BANK_CONFLICT for several patterns:
// ds_read_b128 serves groups of 8 lanes with equal lane bits {0, 1, 4} (the only
// grouping consistent with all of them), ds_read_b64_tr_b16 is consistent with halves
// of 32 lanes.  Under that model:
//  * K reads (lane l: token 16th + (l & 15), chunk 4m + (l >> 4)): a group varies token
//    bits 2, 3 and chunk bit 1 at fixed token parity; s takes t2 and t3 onto position
//    bits 0 and 2, the chunk bit lands on bit 1, so the 8 lanes hit 8 positions.
//  * transpose reads (wide: 4 tokens x 4 chunks x 2 halves; narrow: 4 tokens of
//    consecutive pairs x 2 chunks): within a 32-lane half the token bit that does not
//    give the parity reaches position bit 2 through t1 (and, narrow, t1 and t2 reach
//    bits 1 and 2), so 32 lanes x 8 bytes cover the 64 banks once.
// The previous swizzle (s = the 3-bit reversal of (t >> 1) & 7) was conflict-free under
// a 16-consecutive-lane model and measured 2-way on every K read.  A 1 KiB DMA
// instruction fills 8 consecutive tokens of one 128-byte column; the swizzle only
// permutes 16-byte chunks inside each token's 128 B, so each lane's global offset is a
// per-lane constant plus a wave-uniform term.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int page_swz(int t) {
  return ((t >> 2) & 1) | (((t >> 1) & 1) << 1) | ((((t >> 1) ^ (t >> 2) ^ (t >> 3)) & 1) << 2);
}

// ---------------------------------------------------------------------------
// Number formats
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// OCP e4m3fn encode of a finite float: round to nearest, ties to even; magnitudes
// beyond the largest finite value saturate to +-448; the sign bit is kept.
// Codes are monotonic in magnitude, so rounding into the next binade or from the
// subnormal range into the smallest normal falls out of the integer arithmetic.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  uint32_t bits = __float_as_uint(x);
  uint32_t sign = (bits >> 24) & 0x80u;
  float a = __uint_as_float(bits & 0x7fffffffu);
  uint32_t code;
  if (a >= 0.015625f) {                                  // 2^-6: normal range
    int e = (int)((bits >> 23) & 0xffu) - 127;           // floor(log2 a), a is normal in fp32
    if (e > 8) {
      code = 0x7eu;
    } else {
      float m = __builtin_ldexpf(a, 3 - e);              // in [8, 16), exact scaling
      uint32_t r = (uint32_t)__builtin_rintf(m);         // ties to even; 8..16
      code = ((uint32_t)(e + 7) << 3) + (r - 8u);
      code = code > 0x7eu ? 0x7eu : code;
    }
  } else {
    float m = a * 512.0f;                                // units of 2^-9, exact
    code = (uint32_t)__builtin_rintf(m);                 // 0..8 (8 == smallest normal)
  }
  return sign | code;
}

}  // namespace mla
