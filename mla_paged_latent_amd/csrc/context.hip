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
// Both are pure streaming kernels (HBM-bound) whose consecutive threads cover
// consecutive 16-byte pieces of a row, so loads and stores are contiguous runs.
#include "mla_common.h"
#include "mla_host.h"

namespace mla {


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

// Two adjacent codes (low 16 bits of `two`) times k_scale as a bf16 pair: the
// hardware conversions (e4m3fn -> f32 is exact; f32 -> bf16 rounds to nearest even)
// give the right bits unless a float32 product lies exactly on a bf16 tie, which is
// rare; such a pair is redone with the exact rule above.
__device__ __forceinline__ uint32_t bf16x2_of_products(uint32_t two, float ks) {
#pragma clang fp contract(off)
  const auto v = __builtin_amdgcn_cvt_pk_f32_fp8((int)two, false);
  const float p0 = v[0] * ks, p1 = v[1] * ks;
  const uint32_t b0 = __float_as_uint(p0), b1 = __float_as_uint(p1);
  if (((b0 & 0xFFFFu) == 0x8000u) | ((b1 & 0xFFFFu) == 0x8000u))
    return bf16_of_product(v[0], ks) | (bf16_of_product(v[1], ks) << 16);
  const bf16x2_t r = {(__bf16)p0, (__bf16)p1};
  return *reinterpret_cast<const uint32_t*>(&r);
}

constexpr int kGatherChunks = kRow * 2 / 16;            // 72 output chunks of 8 bf16 per row

// bf16 rows: chunk i of the grid is output row i / 72, bytes 16 (i % 72) .. +15.  Each
// thread takes kGatherUnroll chunks 256 apart per round and runs their dependent loads
// (row -> request -> page id -> data) side by side, so that several chains are in
// flight per thread.
constexpr int kGatherUnroll = 4;

__global__ __launch_bounds__(256) void gather_bf16_kernel(
    const char* __restrict__ pool, int64_t num_pages, const int32_t* __restrict__ block_table,
    int64_t bt_sb, int32_t max_pages, const int32_t* __restrict__ cu_seq_lens,
    const int32_t* __restrict__ seq_starts, const int32_t* __restrict__ token_to_seq, int32_t B,
    int64_t total, uint16_t* __restrict__ out, int64_t out_stride) {
  constexpr int U = kGatherUnroll;
  const int64_t n = total * kGatherChunks;
  const int64_t step = (int64_t)gridDim.x * 256 * U;
  for (int64_t base = (int64_t)blockIdx.x * 256 * U + threadIdx.x; base < n; base += step) {
    int64_t r[U], slot[U];
    int c[U], b[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + 256 * u;
      ok[u] = i < n;
      r[u] = ok[u] ? i / kGatherChunks : 0;
      c[u] = (int)((ok[u] ? i : 0) - r[u] * kGatherChunks);
      b[u] = ok[u] ? token_to_seq[r[u]] : -1;
    }
    // request, logical token and physical page of each row; anything out of range
    // leaves that chunk zero (no access outside the caller's buffers)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      slot[u] = -1;
      if (b[u] >= 0 && b[u] < B) {
        const int64_t j = (int64_t)(seq_starts ? seq_starts[b[u]] : 0) + (r[u] - cu_seq_lens[b[u]]);
        if (j >= 0 && j < (int64_t)max_pages * kPage) slot[u] = j;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (slot[u] >= 0) {
        const int id = block_table[(int64_t)b[u] * bt_sb + (slot[u] >> 6)];
        slot[u] = (id >= 0 && id < num_pages) ? (int64_t)id * kPage + (slot[u] & (kPage - 1)) : -1;
      }
    }
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      v[u] = slot[u] >= 0 ? *reinterpret_cast<const u32x4_t*>(pool + slot[u] * kRowBytesBf16 + c[u] * 16)
                          : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (base + 256 * u < n) *reinterpret_cast<u32x4_t*>(out + r[u] * out_stride + c[u] * 8) = v[u];
  }
}

// fp8 rows: a workgroup gathers blocks of kGatherRows rows.  The row -> request -> page
// chain is walked once per row (one thread each, the results shared through LDS with
// the row's K scale); then every thread issues its share of the block's data loads
// together, with no dependent load in front of them: 9 pieces of 16 codes per thread,
// as two 8-byte loads each (fp8 rows are 584 bytes, so only 8-byte aligned), each
// piece converted to 32 bytes of bf16.  Per-chunk lookup chains as in the bf16 kernel
// above measured 34 us against 28 us for this on the 65,536-row workload; for bf16
// rows, which need no conversion, the chains measured faster (28 vs 31 us).
constexpr int kGatherRows = 64;
constexpr int kGatherPieces = kRow / 16;                 // 36 pieces of 16 codes per row

__global__ __launch_bounds__(256) void gather_fp8_kernel(
    const char* __restrict__ pool, int64_t num_pages, const int32_t* __restrict__ block_table,
    int64_t bt_sb, int32_t max_pages, const int32_t* __restrict__ cu_seq_lens,
    const int32_t* __restrict__ seq_starts, const int32_t* __restrict__ token_to_seq, int32_t B,
    int64_t total, uint16_t* __restrict__ out, int64_t out_stride) {
  constexpr int kPieces = kGatherPieces;
  constexpr int kRows = kGatherRows;
  constexpr int kPerThread = kRows * kPieces / 256;
  static_assert(kRows * kPieces % 256 == 0, "pieces per thread");
  __shared__ int64_t slot_s[kRows];
  __shared__ float scale_s[kRows];
  const int tid = threadIdx.x;
  const int64_t nblk = (total + kRows - 1) / kRows;
  for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    const int64_t r0 = blk * kRows;
    if (tid < kRows) {
      // request, logical token and physical slot of the row; anything out of range
      // leaves the row zero (no access outside the caller's buffers)
      const int64_t r = r0 + tid;
      int64_t slot = -1;
      float ks = 0.f;
      if (r < total) {
        const int b = token_to_seq[r];
        if (b >= 0 && b < B) {
          const int64_t j = (int64_t)(seq_starts ? seq_starts[b] : 0) + (r - cu_seq_lens[b]);
          if (j >= 0 && j < (int64_t)max_pages * kPage) {
            const int id = block_table[(int64_t)b * bt_sb + (j >> 6)];
            if (id >= 0 && id < num_pages) slot = (int64_t)id * kPage + (j & (kPage - 1));
          }
        }
      }
      if (slot >= 0) ks = *reinterpret_cast<const float*>(pool + slot * kRowBytesFp8 + kRow);
      slot_s[tid] = slot;
      scale_s[tid] = ks;
    }
    __syncthreads();
    {
      u32x2_t lo[kPerThread], hi[kPerThread];
#pragma unroll
      for (int k = 0; k < kPerThread; ++k) {
        const int q = tid + 256 * k, row = q / kPieces, c = q % kPieces;
        const int64_t slot = slot_s[row];
        if (slot >= 0) {
          const char* src = pool + slot * kRowBytesFp8 + c * 16;
          lo[k] = *reinterpret_cast<const u32x2_t*>(src);
          hi[k] = *reinterpret_cast<const u32x2_t*>(src + 8);
        } else {
          lo[k] = u32x2_t{0u, 0u};
          hi[k] = u32x2_t{0u, 0u};
        }
      }
#pragma unroll
      for (int k = 0; k < kPerThread; ++k) {
        const int q = tid + 256 * k, row = q / kPieces, c = q % kPieces;
        if (r0 + row >= total) continue;
        const float ks = scale_s[row];
        const uint32_t codes[4] = {lo[k][0], lo[k][1], hi[k][0], hi[k][1]};
        u32x4_t a, b;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          a[m] = bf16x2_of_products(codes[m >> 1] >> (16 * (m & 1)), ks);
          b[m] = bf16x2_of_products(codes[2 + (m >> 1)] >> (16 * (m & 1)), ks);
        }
        uint16_t* dst = out + (r0 + row) * out_stride + c * 16;
        *reinterpret_cast<u32x4_t*>(dst) = a;
        *reinterpret_cast<u32x4_t*>(dst + 8) = b;
      }
    }
    __syncthreads();                                   // the row table is reused by the next block
  }
}

// One thread per 8 elements of a row, kMergeUnroll chunks 256 apart per round (their
// loads in flight together); the row's LSE goes out with its first chunk.
constexpr int kMergeUnroll = 4;

__global__ __launch_bounds__(256) void merge_states_kernel(
    const uint16_t* __restrict__ po, const float* __restrict__ plse, const uint16_t* __restrict__ so,
    const float* __restrict__ slse, int64_t T, int32_t N, int32_t D, int64_t o_st, int64_t o_sh,
    int64_t l_st, int64_t l_sh, uint16_t* __restrict__ out, float* __restrict__ out_lse) {
  constexpr int U = kMergeUnroll;
  const int cpr = D >> 3;                                 // chunks per row
  const int64_t n = T * N * cpr;
  const int64_t step = (int64_t)gridDim.x * 256 * U;
  for (int64_t base = (int64_t)blockIdx.x * 256 * U + threadIdx.x; base < n; base += step) {
    int64_t off[U], loff[U];
    int c[U];
    float lp[U], ls[U];
    u32x4_t a[U], bb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + 256 * u < n ? base + 256 * u : n - 1;   // clamped: in bounds, not stored
      const int64_t row = i / cpr;
      c[u] = (int)(i - row * cpr);
      const int64_t t = row / N;
      const int h = (int)(row - t * N);
      loff[u] = t * l_st + h * l_sh;
      off[u] = t * o_st + h * o_sh + 8 * c[u];
      lp[u] = plse[loff[u]];
      ls[u] = slse[loff[u]];
      a[u] = *reinterpret_cast<const u32x4_t*>(po + off[u]);
      bb[u] = *reinterpret_cast<const u32x4_t*>(so + off[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float m = fmaxf(lp[u], ls[u]);
      u32x4_t v = {0u, 0u, 0u, 0u};
      float lse = -INFINITY;
      if (m != -INFINITY) {
        const float wp = expf(lp[u] - m), ws = expf(ls[u] - m);   // exp(-inf) = 0: an empty state weighs nothing
        const float wsum = wp + ws;
        const float fp = wp / wsum, fs = ws / wsum;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float x0 = fp * bf16_bits_to_f32(a[u][k] & 0xFFFFu) + fs * bf16_bits_to_f32(bb[u][k] & 0xFFFFu);
          const float x1 = fp * bf16_bits_to_f32(a[u][k] >> 16) + fs * bf16_bits_to_f32(bb[u][k] >> 16);
          const bf16x2_t p = {(__bf16)x0, (__bf16)x1};
          v[k] = *reinterpret_cast<const uint32_t*>(&p);
        }
        lse = m + logf(wsum);
      }
      if (base + 256 * u < n) {
        *reinterpret_cast<u32x4_t*>(out + off[u]) = v;
        if (out_lse && c[u] == 0) out_lse[loff[u]] = lse;
      }
    }
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
  if (kv_dtype == MLA_KV_BF16) {
    const unsigned grid = stream_grid((total_rows * kGatherChunks + kGatherUnroll - 1) / kGatherUnroll, di);
    hipLaunchKernelGGL(gather_bf16_kernel, dim3(grid), dim3(256), 0, s, (const char*)kv_cache, num_pages,
                       block_table, bt_stride_b, max_pages_per_seq, cu_seq_lens, seq_starts, token_to_seq, B,
                       total_rows, (uint16_t*)out, out_stride);
  } else {
    const int64_t row_blocks = (total_rows + kGatherRows - 1) / kGatherRows;
    const unsigned grid = (unsigned)(row_blocks < 1048576 ? row_blocks : 1048576);
    hipLaunchKernelGGL(gather_fp8_kernel, dim3(grid), dim3(256), 0, s, (const char*)kv_cache, num_pages,
                       block_table, bt_stride_b, max_pages_per_seq, cu_seq_lens, seq_starts, token_to_seq, B,
                       total_rows, (uint16_t*)out, out_stride);
  }
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
  const unsigned grid = stream_grid((T * N * (D >> 3) + kMergeUnroll - 1) / kMergeUnroll, di);
  hipLaunchKernelGGL(merge_states_kernel, dim3(grid), dim3(256), 0, s, (const uint16_t*)prefix_out, prefix_lse,
                     (const uint16_t*)suffix_out, suffix_lse, T, N, D, o_stride_t, o_stride_h, lse_stride_t,
                     lse_stride_h, (uint16_t*)out, out_lse);
  return launch_status();
}
