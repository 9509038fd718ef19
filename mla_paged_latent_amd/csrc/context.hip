// The two steps either side of decode in chunked prefill:
//   mla_gather_cache       context rows of the paged cache -> one contiguous bf16
//                          workspace (fp8 rows upconverted on the way)
//   mla_merge_attn_states  two attention states of the same query rows over
//                          disjoint key sets -> one state
// Source: "vLLM 源码完全拆解(三十七):MLA 注意力后端", §Prefill (chunked context:
// the gather by block_table / cu_seq_lens / token_to_seq into a workspace for
// kv_b_proj, fp8 upconverted to bf16, chunk starts on page boundaries; and
// merge_attn_states, re-weighting by exp(lse - max_lse) with empty states at
// weight zero).
//
// Both are pure streaming kernels (HBM-bound): one thread per 16 output bytes, so
// a row's threads are consecutive and every load and store is a whole 16-byte (fp8
// codes: 8-byte) piece of a contiguous row.
#include "mla_common.h"
#include "mla_host.h"

namespace mla {

constexpr int kGatherChunks = kRow * 2 / 16;            // 72 output chunks of 8 bf16 per row

// Value of an OCP e4m3fn code (exact in float32): exponent field 0 is subnormal,
// S.1111.111 is NaN, bias 7.
__device__ __forceinline__ float e4m3_value_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  float mag = e == 0 ? (float)m * 0.001953125f                        // m * 2^-9
                     : __uint_as_float(((e + 120u) << 23) | (m << 20));  // (1 + m/8) 2^(e-7)
  if (e == 15u && m == 7u) mag = __uint_as_float(0x7FC00000u);
  return (c & 0x80u) ? -mag : mag;
}

// bfloat16 bits of the exact product v * s, rounded once (nearest, ties to even).
// v has at most 4 significant bits, so v * s has at most 28: p = fl(v * s) holds the
// top 24 and fma(v, s, -p) the exact rest.  Rounding p to bf16 is right unless p sits
// exactly halfway between two bf16 values; there the sign of the rest decides (exact
// for products of magnitude >= 2^-126; below that the rest can round to zero and the
// tie rule is applied instead).
__device__ __forceinline__ uint32_t bf16_of_product(float v, float s) {
#pragma clang fp contract(off)
  const float p = v * s;
  const uint32_t pb = __float_as_uint(p);
  if (p != p) return ((pb >> 16) & 0x8000u) | 0x7FC0u;
  uint32_t r = (pb + 0x7FFFu + ((pb >> 16) & 1u)) >> 16;
  if ((pb & 0xFFFFu) == 0x8000u) {
    const float rest = __builtin_fmaf(v, s, -p);
    if (rest != 0.f) r = (pb >> 16) + (((rest > 0.f) == (p > 0.f)) ? 1u : 0u);
  }
  return r & 0xFFFFu;
}

template <bool FP8>
__global__ __launch_bounds__(256) void gather_cache_kernel(
    const char* __restrict__ pool, int64_t num_pages, const int32_t* __restrict__ block_table,
    int64_t bt_sb, int32_t max_pages, const int32_t* __restrict__ cu_seq_lens,
    const int32_t* __restrict__ seq_starts, const int32_t* __restrict__ token_to_seq, int32_t B,
    int64_t total, uint16_t* __restrict__ out, int64_t out_stride) {
  const int64_t n = total * kGatherChunks;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / kGatherChunks;
    const int c = (int)(i - r * kGatherChunks);
    u32x4_t v = {0u, 0u, 0u, 0u};
    // request, logical token and physical page of this row; anything out of range
    // leaves the row's chunk zero (no access outside the caller's buffers)
    const int b = token_to_seq[r];
    if (b >= 0 && b < B) {
      const int64_t j = (int64_t)(seq_starts ? seq_starts[b] : 0) + (r - cu_seq_lens[b]);
      if (j >= 0 && j < (int64_t)max_pages * kPage) {
        const int id = block_table[(int64_t)b * bt_sb + (j >> 6)];
        if (id >= 0 && id < num_pages) {
          const int64_t slot = (int64_t)id * kPage + (j & (kPage - 1));
          if constexpr (!FP8) {
            v = *reinterpret_cast<const u32x4_t*>(pool + slot * kRowBytesBf16 + c * 16);
          } else {
            const char* row = pool + slot * kRowBytesFp8;
            const u32x2_t codes = *reinterpret_cast<const u32x2_t*>(row + c * 8);
            const float ks = *reinterpret_cast<const float*>(row + kRow);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const uint32_t w = codes[k >> 1] >> (16 * (k & 1));
              v[k] = bf16_of_product(e4m3_value_f32(w & 0xFFu), ks) |
                     (bf16_of_product(e4m3_value_f32((w >> 8) & 0xFFu), ks) << 16);
            }
          }
        }
      }
    }
    *reinterpret_cast<u32x4_t*>(out + r * out_stride + c * 8) = v;
  }
}

// One thread per 8 elements of a row; the row's LSE goes out with its first chunk.
__global__ __launch_bounds__(256) void merge_states_kernel(
    const uint16_t* __restrict__ po, const float* __restrict__ plse, const uint16_t* __restrict__ so,
    const float* __restrict__ slse, int64_t T, int32_t N, int32_t D, int64_t o_st, int64_t o_sh,
    int64_t l_st, int64_t l_sh, uint16_t* __restrict__ out, float* __restrict__ out_lse) {
  const int cpr = D >> 3;                                 // chunks per row
  const int64_t n = T * N * cpr;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t row = i / cpr;
    const int c = (int)(i - row * cpr);
    const int64_t t = row / N;
    const int h = (int)(row - t * N);
    const float lp = plse[t * l_st + h * l_sh], ls = slse[t * l_st + h * l_sh];
    const int64_t off = t * o_st + h * o_sh + 8 * c;
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(po + off);
    const u32x4_t bb = *reinterpret_cast<const u32x4_t*>(so + off);
    const float m = fmaxf(lp, ls);
    u32x4_t v = {0u, 0u, 0u, 0u};
    float lse = -INFINITY;
    if (m != -INFINITY) {
      const float wp = expf(lp - m), ws = expf(ls - m);   // exp(-inf) = 0: an empty state weighs nothing
      const float wsum = wp + ws;
      const float fp = wp / wsum, fs = ws / wsum;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float x0 = fp * bf16_bits_to_f32(a[k] & 0xFFFFu) + fs * bf16_bits_to_f32(bb[k] & 0xFFFFu);
        const float x1 = fp * bf16_bits_to_f32(a[k] >> 16) + fs * bf16_bits_to_f32(bb[k] >> 16);
        const bf16x2_t p = {(__bf16)x0, (__bf16)x1};
        v[k] = *reinterpret_cast<const uint32_t*>(&p);
      }
      lse = m + logf(wsum);
    }
    *reinterpret_cast<u32x4_t*>(out + off) = v;
    if (out_lse && c == 0) out_lse[t * l_st + h * l_sh] = lse;
  }
}

inline unsigned stream_grid(int64_t threads, const DeviceInfo& di) {
  const int64_t blocks = (threads + 255) / 256;
  const int64_t cap = (int64_t)di.cu_count * 16;          // enough waves in flight per CU
  return (unsigned)(blocks < cap ? (blocks > 0 ? blocks : 1) : cap);
}

}  // namespace mla

extern "C" mla_status_t mla_gather_cache(const void* kv_cache, int32_t kv_dtype, int64_t num_pages,
                                         const int32_t* block_table, int64_t bt_stride_b,
                                         int32_t max_pages_per_seq, const int32_t* cu_seq_lens,
                                         const int32_t* seq_starts, const int32_t* token_to_seq,
                                         int32_t B, int64_t total_rows, void* out, int64_t out_stride,
                                         void* stream) {
  using namespace mla;
  if (kv_dtype != MLA_KV_BF16 && kv_dtype != MLA_KV_FP8_E4M3) return MLA_ERR_DTYPE;
  if (total_rows < 0 || B < 1 || num_pages < 1 || max_pages_per_seq < 1 || bt_stride_b < max_pages_per_seq)
    return MLA_ERR_SHAPE;
  if (total_rows == 0) return MLA_OK;
  if (out_stride < kRow || total_rows > ((int64_t)1 << 40)) return MLA_ERR_SHAPE;
  if (!kv_cache || !block_table || !cu_seq_lens || !token_to_seq || !out) return MLA_ERR_NULL;
  if (!aligned16(kv_cache) || !aligned16(out) || !mult8(out_stride) ||
      (reinterpret_cast<uintptr_t>(block_table) & 3u) || (reinterpret_cast<uintptr_t>(cu_seq_lens) & 3u) ||
      (reinterpret_cast<uintptr_t>(token_to_seq) & 3u) || (reinterpret_cast<uintptr_t>(seq_starts) & 3u))
    return MLA_ERR_ALIGN;
  if (max_pages_per_seq > 0x7fffffff / kPage) max_pages_per_seq = 0x7fffffff / kPage;
  DeviceInfo di;
  mla_status_t st = device_info(&di);
  if (st != MLA_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const unsigned grid = stream_grid(total_rows * kGatherChunks, di);
  if (kv_dtype == MLA_KV_BF16)
    hipLaunchKernelGGL(gather_cache_kernel<false>, dim3(grid), dim3(256), 0, s, (const char*)kv_cache, num_pages,
                       block_table, bt_stride_b, max_pages_per_seq, cu_seq_lens, seq_starts, token_to_seq, B,
                       total_rows, (uint16_t*)out, out_stride);
  else
    hipLaunchKernelGGL(gather_cache_kernel<true>, dim3(grid), dim3(256), 0, s, (const char*)kv_cache, num_pages,
                       block_table, bt_stride_b, max_pages_per_seq, cu_seq_lens, seq_starts, token_to_seq, B,
                       total_rows, (uint16_t*)out, out_stride);
  return launch_status();
}

extern "C" mla_status_t mla_merge_attn_states(const void* prefix_out, const float* prefix_lse,
                                              const void* suffix_out, const float* suffix_lse, int64_t T,
                                              int32_t N, int32_t D, int64_t o_stride_t, int64_t o_stride_h,
                                              int64_t lse_stride_t, int64_t lse_stride_h, void* out,
                                              float* out_lse, void* stream) {
  using namespace mla;
  if (T < 0 || N < 1 || D < 8 || (D & 7) || D > 4096) return MLA_ERR_SHAPE;
  if (T == 0) return MLA_OK;
  if (T > ((int64_t)1 << 40) / N) return MLA_ERR_SHAPE;
  if (!prefix_out || !prefix_lse || !suffix_out || !suffix_lse || !out) return MLA_ERR_NULL;
  if (!aligned16(prefix_out) || !aligned16(suffix_out) || !aligned16(out) || !mult8(o_stride_t) ||
      !mult8(o_stride_h) || (reinterpret_cast<uintptr_t>(prefix_lse) & 3u) ||
      (reinterpret_cast<uintptr_t>(suffix_lse) & 3u) || (reinterpret_cast<uintptr_t>(out_lse) & 3u))
    return MLA_ERR_ALIGN;
  DeviceInfo di;
  mla_status_t st = device_info(&di);
  if (st != MLA_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const unsigned grid = stream_grid(T * N * (D >> 3), di);
  hipLaunchKernelGGL(merge_states_kernel, dim3(grid), dim3(256), 0, s, (const uint16_t*)prefix_out, prefix_lse,
                     (const uint16_t*)suffix_out, suffix_lse, T, N, D, o_stride_t, o_stride_h, lse_stride_t,
                     lse_stride_h, (uint16_t*)out, out_lse);
  return launch_status();
}
