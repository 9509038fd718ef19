// The row writer of mla_cache_write, shared by its own kernel and by the launch that
// runs it beside the query absorption (mla_absorb_q_cache_write).
// Source: "vLLM 源码完全拆解(三十七):MLA 注意力后端", §写缓存 (latent and k_pe written
// into one row per token at slot_mapping[t]) and §缓存的形状 (576-element rows; fp8 rows
// carry one float32 scale for K and one for V, 584 bytes).
#pragma once
#include "mla_common.h"
#include "mla_host.h"

namespace mla {

// Token t's row, written by one wave (lane l holds latent elements 8l .. 8l+7, lanes
// 0..7 also rope elements 8l .. 8l+7); t < T is the caller's check.
template <bool FP8>
__device__ __forceinline__ void cache_write_row(const uint16_t* __restrict__ kv_c, int64_t kv_stride,
                                                const uint16_t* __restrict__ k_pe, int64_t pe_stride,
                                                const int64_t* __restrict__ slots, char* __restrict__ pool,
                                                int64_t num_pages, int64_t t, int l) {
  // the slot and the row are read together (no load waits for another): lanes 8..63
  // re-read one of the 8 rope chunks and drop it
  const int64_t slot = slots[t];
  const uint4* src_c = reinterpret_cast<const uint4*>(kv_c + t * kv_stride);
  const uint4* src_p = reinterpret_cast<const uint4*>(k_pe + t * pe_stride);
  const uint4 vc = src_c[l];                      // latent elements 8l .. 8l+7
  const uint4 vp_any = src_p[l & 7];
  const uint4 vp = l < 8 ? vp_any : make_uint4(0, 0, 0, 0);   // rope elements 8l .. 8l+7
  if (slot < 0 || slot >= num_pages * kPage) return;   // padding or out of range: skip

  if constexpr (!FP8) {
    uint4* dst = reinterpret_cast<uint4*>(pool + slot * kRowBytesBf16);
    dst[l] = vc;
    if (l < 8) dst[64 + l] = vp;
  } else {
    // per-token amax over the 576 values
    const uint32_t wc[4] = {vc.x, vc.y, vc.z, vc.w};
    const uint32_t wp[4] = {vp.x, vp.y, vp.z, vp.w};
    float xc[8], xp[8];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xc[2 * i] = bf16_bits_to_f32(wc[i] & 0xffffu);
      xc[2 * i + 1] = bf16_bits_to_f32(wc[i] >> 16);
      xp[2 * i] = bf16_bits_to_f32(wp[i] & 0xffffu);
      xp[2 * i + 1] = bf16_bits_to_f32(wp[i] >> 16);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fmaxf(fabsf(xc[i]), fabsf(xp[i])));
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, shfl_xor_f(amax, m));
    float s = __fdiv_rn(amax, 448.0f);
    if (s == 0.f) s = 1.f;
    uint32_t lo = 0, hi = 0, plo = 0, phi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= e4m3_encode(__fdiv_rn(xc[i], s)) << (8 * i);
      hi |= e4m3_encode(__fdiv_rn(xc[4 + i], s)) << (8 * i);
      plo |= e4m3_encode(__fdiv_rn(xp[i], s)) << (8 * i);
      phi |= e4m3_encode(__fdiv_rn(xp[4 + i], s)) << (8 * i);
    }
    char* row = pool + slot * kRowBytesFp8;           // 8-byte aligned (584 = 8 * 73)
    reinterpret_cast<uint2*>(row)[l] = make_uint2(lo, hi);
    if (l < 8) reinterpret_cast<uint2*>(row + kLatent)[l] = make_uint2(plo, phi);
    if (l == 0) reinterpret_cast<float2*>(row + kRow)[0] = make_float2(s, s);
  }
}

// The argument checks of mla_cache_write (MLA_OK when T == 0 with any pointers).
inline mla_status_t cache_write_check(const void* kv_c, int64_t kv_c_stride_t, const void* k_pe,
                                      int64_t k_pe_stride_t, const int64_t* slot_mapping, int64_t T,
                                      const void* kv_cache, int32_t kv_dtype, int64_t num_pages) {
  if (kv_dtype != MLA_KV_BF16 && kv_dtype != MLA_KV_FP8_E4M3) return MLA_ERR_DTYPE;
  if (T < 0 || num_pages < 0) return MLA_ERR_SHAPE;
  if (T == 0) return MLA_OK;
  if (!kv_c || !k_pe || !slot_mapping || !kv_cache) return MLA_ERR_NULL;
  if (kv_c_stride_t < kLatent || k_pe_stride_t < kRope) return MLA_ERR_SHAPE;
  if (!aligned16(kv_c) || !aligned16(k_pe) || !aligned16(kv_cache) || !mult8(kv_c_stride_t) ||
      !mult8(k_pe_stride_t))
    return MLA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(slot_mapping) & 7u) != 0) return MLA_ERR_ALIGN;
  return MLA_OK;
}

}  // namespace mla
