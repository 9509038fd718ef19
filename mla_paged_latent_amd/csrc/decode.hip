// mla_decode: paged split-KV absorbed-MQA decode over 576-element latent rows,
// with a device-side split planner and an LSE merge of the splits.
//
// Sources: "vLLM 源码完全拆解(三十七):MLA 注意力后端" -- §两套算法 (decode as MQA over
// [kv_c | k_pe] with kv_c doubling as V; scale stays 1/sqrt(192)), §FlashMLA (one KV
// head shared by all query heads, 64-token pages, a per-sequence split plan built
// from seq_lens, single-partition batch-invariant mode), §Triton MLA (split partials
// of 512 outputs + 1 LSE in float32, a second stage reduces them; causality of a
// multi-token query through per-row visible lengths), §Prefill (merge_attn_states:
// partials re-weighted by exp(lse - max), empty partials o = 0, lse = -inf);
// "Triton und MLA", §Datenfluss and §Entwurfsmotivation (natural-log LSE returned).
//
// Structure (all on the caller's stream, no host synchronisation):
//   plan_kernel   one workgroup: per-request split count and page-aligned token
//                 ranges -> (request, split) pair table in the workspace
//   decode_kernel persistent grid: one work unit = (pair, head group); the unit's
//                 pages stream through LDS (double-buffered global->LDS DMA), every
//                 query head of the group scores against each staged page:
//                   S^T = K . Q^T  (MFMA; Q lives in registers as the B operand)
//                   online softmax in the log2 domain, per head = per lane
//                   O^T += V^T . P^T (MFMA; V^T via LDS transpose reads, P^T is the
//                                     S^T accumulator re-packed to bf16 in place)
//                 then writes the final output (single split) or a float32 partial
//   merge_kernel  LSE-weighted combine of the partials of split requests
#include <utility>

#include "mla_common.h"
#include "mla_host.h"

namespace mla {

struct DecodeParams {
  const uint16_t* q;
  int64_t q_sb, q_st, q_sh;
  const char* kv;
  int64_t num_pages;
  const int32_t* block_table;
  int64_t bt_sb;
  int32_t max_pages;
  const int32_t* seq_lens;
  int32_t B, q_len, N;
  int32_t n_hg;        // head groups per request
  int32_t m_wg;        // query rows per work unit (16 narrow, 128 wide)
  int32_t hg_heads;    // heads per head group = m_wg / q_len
  float scale_log2;    // softmax_scale * log2(e)
  uint16_t* out;
  int64_t o_sb, o_st, o_sh;
  float* lse;
  // workspace views
  int32_t* hdr;        // [0] pairs, [1] units
  int4* req;           // per request: {first pair, splits, chunk, clamped seq_len}
  int4* pairs;         // per pair: {request, split, token begin, token end}
  float* part_lse;     // [pairs * n_hg * m_wg]
  float* part_o;       // [pairs * n_hg * m_wg * 512]
  int32_t max_pairs;
  int32_t num_splits;  // 0 auto, 1 single, k forced
  int32_t target_pairs;
};

// unit -> (pair, head group).  Sibling head groups of one pair sit 8 units apart so
// that, with a grid that is a multiple of 8, they run at the same time on the same
// XCD (workgroups are dispatched round-robin over the 8 XCDs) and share the pair's
// pages through that XCD's L2.
__device__ __forceinline__ void unit_to_pair(int u, int n_hg, int* pair, int* hg) {
  if (n_hg == 1) {
    *pair = u;
    *hg = 0;
  } else {
    *pair = (u / (8 * n_hg)) * 8 + (u & 7);
    *hg = (u >> 3) % n_hg;
  }
}

// ---------------------------------------------------------------------------
// Split planner
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void plan_kernel(DecodeParams p) {
  __shared__ long long red[256];
  __shared__ int scan[256];
  const int tid = threadIdx.x;
  const int seq_cap = p.max_pages * kPage;
  long long local = 0;
  for (int b = tid; b < p.B; b += 256) {
    int s = p.seq_lens[b];
    s = s < 0 ? 0 : (s > seq_cap ? seq_cap : s);
    local += s;
  }
  red[tid] = local;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  const long long total = red[0];
  // automatic mode: one common page-aligned chunk so that the whole batch makes
  // about target_pairs (request, split) pairs
  long long auto_chunk = (total + p.target_pairs - 1) / p.target_pairs;
  auto_chunk = ((auto_chunk + kPage - 1) / kPage) * kPage;
  if (auto_chunk < kPage) auto_chunk = kPage;

  int base = 0;
  for (int b0 = 0; b0 < p.B; b0 += 256) {
    const int b = b0 + tid;
    int ns = 0, chunk = kPage, s = 0;
    if (b < p.B) {
      s = p.seq_lens[b];
      s = s < 0 ? 0 : (s > seq_cap ? seq_cap : s);
      long long c;
      if (p.num_splits == 0)
        c = auto_chunk;
      else if (p.num_splits == 1)
        c = s > 0 ? s : 1;
      else
        c = (s + p.num_splits - 1) / p.num_splits;
      c = ((c + kPage - 1) / kPage) * kPage;
      if (c < kPage) c = kPage;
      chunk = (int)c;
      ns = s > 0 ? (int)((s + c - 1) / c) : 1;
    }
    // exclusive scan of ns over the 256 requests of this block
    scan[tid] = ns;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
      const int v = tid >= o ? scan[tid - o] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const int incl = scan[tid];
    const int block_total = scan[255];
    if (b < p.B) {
      const int first = base + incl - ns;
      p.req[b] = make_int4(first, ns, chunk, s);
      for (int k = 0; k < ns; ++k) {
        const int pi = first + k;
        if (pi < p.max_pairs) {
          const int t0 = k * chunk;
          const int t1 = (k + 1) * chunk < s ? (k + 1) * chunk : s;
          p.pairs[pi] = make_int4(b, k, t0, t1 > t0 ? t1 : t0);
        }
      }
    }
    base += block_total;
    __syncthreads();
  }
  if (tid == 0) {
    const int P = base < p.max_pairs ? base : p.max_pairs;
    p.hdr[0] = P;
    p.hdr[1] = p.n_hg == 1 ? P : ((P + 7) / 8) * 8 * p.n_hg;
  }
}

// ---------------------------------------------------------------------------
// Page staging
// ---------------------------------------------------------------------------
// bf16 page: 72 DMA instructions of 64 x 16 B; wave w issues instructions w, w+4, ...
// (18 per wave).  Instruction k fills LDS group k >> 3 for tokens 8*(k & 7) + (lane >> 3);
// lane j loads global chunk 8*(k >> 3) + ((j & 7) ^ s(j >> 3)) of that token (the
// swizzle only sees t & 7 = j >> 3), i.e. page + lane_off + 9216*(k & 7) + 128*(k >> 3).
template <int... I>
__device__ __forceinline__ void issue_bf16_seq(std::integer_sequence<int, I...>, const char* page,
                                               const char* half1, uint32_t voff, uint32_t lds) {
  (dma_16B<128 * (I >> 1), 4096 * I>((I & 1) ? half1 : page, voff, lds), ...);
}

__device__ __forceinline__ void issue_page_bf16(const char* page, MLA_LDS char* dst, int w, int l) {
  // instruction k = w + 4i covers tokens 8*(k & 7) .. +7 of 128-byte column k >> 3;
  // with w < 4 that is tokens 8w + 32*(i & 1) and column i >> 1, so the wave's part
  // of the offset sits in voff and the rest is a compile-time constant.
  const uint32_t voff = (uint32_t)((l >> 3) * kRowBytesBf16 + ((l & 7) ^ page_swz(l >> 3)) * 16 +
                                   w * 8 * kRowBytesBf16);
  const char* half1 = page + 32 * kRowBytesBf16;
  const uint32_t lds = lds_addr(dst) + (uint32_t)w * 1024u;
  issue_bf16_seq(std::make_integer_sequence<int, 18>{}, page, half1, voff, lds);
}

// fp8 page: the 37376 raw bytes (16-byte aligned) as 2336 flat 16-B chunks in 37
// instructions k = w + 4i; wave 0 issues 10 of them (the last one half-masked),
// waves 1..3 issue 9.
template <int I>
__device__ __forceinline__ void issue_fp8_one(const char* page, uint32_t voff, uint32_t lds, int w, int l) {
  const int k = w + 4 * I;
  if (k < 37 && k * 64 + l < kPageBytesFp8 / 16) dma_16B<0, 4096 * I>(page + 4096 * I, voff, lds);
}

template <int... I>
__device__ __forceinline__ void issue_fp8_seq(std::integer_sequence<int, I...>, const char* page, uint32_t voff,
                                              uint32_t lds, int w, int l) {
  (issue_fp8_one<I>(page, voff, lds, w, l), ...);
}

__device__ __forceinline__ void issue_page_fp8(const char* page, MLA_LDS char* dst, int w, int l) {
  const uint32_t voff = (uint32_t)(w * 1024 + l * 16);
  const uint32_t lds = lds_addr(dst) + (uint32_t)w * 1024u;
  issue_fp8_seq(std::make_integer_sequence<int, 10>{}, page, voff, lds, w, l);
}

// Physical page ids of a unit, 64 at a time: lane j of every wave holds the id of
// logical page base + j in one VGPR and the id of page pg is read with readlane, so a
// page's DMA never waits on a block-table load (the ids are fetched up to 64 pages
// ahead; the reload every 64 pages is the only exposed table access).
struct PageIds {
  int base;   // logical page held by lane 0
  int vec;    // this lane's id (clamped into [0, num_pages))
};

__device__ __forceinline__ void load_page_ids(PageIds& ids, const DecodeParams& p, int b, int base,
                                              int pg_end, int l) {
  ids.base = base;
  int id = 0;
  if (base + l < pg_end) id = p.block_table[(int64_t)b * p.bt_sb + base + l];
  ids.vec = (id < 0 || id >= p.num_pages) ? 0 : id;     // out-of-contract id: clamp, never fault
}

__device__ __forceinline__ const char* page_ptr(PageIds& ids, const DecodeParams& p, int b, int pg,
                                                int pg_end, int l, bool fp8) {
  if (pg - ids.base >= 64) load_page_ids(ids, p, b, pg, pg_end, l);   // uniform branch
  const int id = __builtin_amdgcn_readlane(ids.vec, pg - ids.base);
  return p.kv + (int64_t)id * (fp8 ? kPageBytesFp8 : kPageBytesBf16);
}

// ---------------------------------------------------------------------------
// LDS plan
// ---------------------------------------------------------------------------
//   bf16: two swizzled pages [0, 73728) and [73728, 147456)
//   fp8 : raw pages at 0 and 37376, converted bf16 page at 74752, k/v scales after
constexpr int kLdsBf16 = 2 * kPageBytesBf16;
constexpr int kFp8Raw0 = 0;
constexpr int kFp8Raw1 = kPageBytesFp8;
constexpr int kFp8Conv = 2 * kPageBytesFp8;
constexpr int kFp8KScale = kFp8Conv + kPageBytesBf16;
constexpr int kFp8VScale = kFp8KScale + 256;
constexpr int kFp8IVScale = kFp8VScale + 256;
constexpr int kLdsFp8 = kFp8IVScale + 256;
constexpr int kLdsPages = kLdsBf16 > kLdsFp8 ? kLdsBf16 : kLdsFp8;
constexpr int kLdsFlag = kLdsPages;                    // overflow flag of the reference max
constexpr int kLdsBytes = kLdsPages + 16;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");

// fp8 raw page -> swizzled bf16 page (exact: every e4m3fn value is a bf16 value);
// token rows at or past `valid` become zero so stale pool bytes never reach the MFMA.
__device__ __forceinline__ void convert_fp8_page(const MLA_LDS char* raw, MLA_LDS char* conv,
                                                 MLA_LDS float* ks, MLA_LDS float* vs,
                                                 MLA_LDS float* ivs, int valid, int tid,
                                                 float scale_log2) {
  // not unrolled: the query fragments and accumulators are live across this loop
#pragma unroll 1
  for (int s = tid; s < kPage * kChunksPerRow; s += 256) {
    const int t = (s >> 3) & 63;
    const int c = (s >> 9) * 8 + ((s & 7) ^ page_swz(t));
    bf16x8_t v = {};
    if (t < valid) {
      const u32x2_t code = *reinterpret_cast<const MLA_LDS u32x2_t*>(raw + t * kRowBytesFp8 + c * 8);
      const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)code[0], 1.0f, false);
      const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)code[0], 1.0f, true);
      const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)code[1], 1.0f, false);
      const bf16x2_t e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)code[1], 1.0f, true);
      v = bf16x8_t{a[0], a[1], b[0], b[1], d[0], d[1], e[0], e[1]};
    }
    *reinterpret_cast<MLA_LDS bf16x8_t*>(conv + s * 16) = v;
  }
  if (tid < kPage) {
    float k = 0.f, v = 0.f;
    if (tid < valid) {
      const f32x2_t sc = *reinterpret_cast<const MLA_LDS f32x2_t*>(raw + tid * kRowBytesFp8 + kRow);
      k = sc[0];
      v = sc[1];
    }
    ks[tid] = k * scale_log2;                          // k_scale folded with the softmax scale
    vs[tid] = v;
    ivs[tid] = v != 0.f ? 1.0f / v : 0.f;
  }
}

__device__ __forceinline__ void zero_tail_rows(MLA_LDS char* page, int valid, int tid) {
  const int per_group = (kPage - valid) * 8;          // slots of rows valid..63 in one group
  for (int s = tid; s < 9 * per_group; s += 256) {
    const int grp = s / per_group;
    const int slot = grp * kGroupSlots + valid * 8 + (s - grp * per_group);
    *reinterpret_cast<MLA_LDS u32x4_t*>(page + slot * 16) = u32x4_t{0u, 0u, 0u, 0u};
  }
}

// ---------------------------------------------------------------------------
// Per-unit compute: wide variant (128 query rows, 32 per wave, 32x32x16 MFMA)
// ---------------------------------------------------------------------------
// Softmax bookkeeping without rescaling the accumulators.  Each row's reference
// max m is fixed from the first 32-token block of the unit (exact for that block);
// later scores may exceed it, so p = 2^(s - m) can be > 1, which float32
// accumulation and bfloat16 probabilities represent without loss of relative
// precision.  A visible score more than kRefSlack above m would risk overflow:
// the block then raises a flag and the workgroup redoes the unit with the larger
// reference.  O never needs a VALU rescale inside the page loop.
constexpr float kRefSlack = 64.0f;

struct WideState {
  f32x16_t o[16];     // O^T: 16 blocks of 32 latent features x 32 rows (lane = row)
  float m;            // reference max (log2 domain), -inf until set
  float l;            // sum of p over this lane's half of the tokens (for the LSE)
  float lr;           // same sum over the bf16-rounded weights (normalises O)
  float m_seen;       // largest visible score seen (for a restart)
};

template <bool FP8>
__device__ __forceinline__ void wide_page(const MLA_LDS char* pg, const MLA_LDS float* ks,
                                          const MLA_LDS float* vs, const MLA_LDS float* ivs,
                                          const bf16x8_t (&qf)[36],
                                          WideState& st, int tok0, int nvis, bool need_mask,
                                          float scale_log2, int l, bool first,
                                          MLA_LDS int* overflow) {
  const int h32 = l >> 5, c32 = l & 31;
  const int g = l >> 4, lg = l & 15;
  // K chunk c = 2*kk + h32 of token 32*tb + c32: group kk >> 2, in-group chunk
  // 2*(kk & 3) + h32, swizzle s(c32) (the swizzle sees t & 7 only).
  uint32_t kbase[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) kbase[m] = (uint32_t)(c32 * 8 + ((2 * m + h32) ^ page_swz(c32))) * 16;
  // Transpose reads: the 16-lane group g reads tokens 16u + 8r + 4*h32 + e (e = 0..3,
  // read r = 0/1) at features 32*fb + 16*(g & 1) + [0, 16); lane lg supplies token row
  // lg >> 2 and column 4*(lg & 3).  Chunk c = 4*fb + cpart lies in group fb >> 1 at
  // in-group chunk 4*(fb & 1) + cpart and the swizzle sees t & 7 = 4*h32 + (lg >> 2).
  const int vt = 4 * h32 + (lg >> 2);
  const int cpart = 2 * (g & 1) + ((lg & 3) >> 1);
  uint32_t vbase[2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
    vbase[m] = (uint32_t)(vt * 8 + ((4 * m + cpart) ^ page_swz(vt))) * 16 + (uint32_t)(lg & 1) * 8;

  // The page is processed as two 32-token halves, each a full online-softmax step.
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    // S^T = K . Q^T over 576 features in 36 steps of 16.  K fragments are read
    // kPrefK steps ahead of their MFMA (a rolling register buffer) so the LDS latency
    // hides behind the MFMA pipeline; the scheduler is told to alternate one LDS read
    // with one MFMA.
    constexpr int kPrefK = 4;
    const uint32_t kofs = tb * (32 * 8 * 16);
    bf16x8_t kbuf[kPrefK];
#pragma unroll
    for (int d = 0; d < kPrefK; ++d) kbuf[d] = lds_read_b128(pg, kbase[d & 3] + (d >> 2) * kGroupBytes + kofs);
    __builtin_amdgcn_sched_group_barrier(0x100, kPrefK, 0);               // prologue reads first
    f32x16_t sc = {};
#pragma unroll
    for (int kk = 0; kk < 36; ++kk) {
      const bf16x8_t a = kbuf[kk % kPrefK];
      const int nk = kk + kPrefK;
      if (nk < 36) kbuf[kk % kPrefK] = lds_read_b128(pg, kbase[nk & 3] + (nk >> 2) * kGroupBytes + kofs);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], sc, 0, 0, 0);
      if (nk < 36) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                // MFMA
    }
    // scores -> log2 domain, mask, tile max.  Element i = 4a + j is token
    // 32*tb + 8a + 4*h32 + j of the page.  For fp8 the per-token factors (k_scale *
    // softmax scale, v_scale, 1/v_scale) of the 4 tokens of group a are read as one
    // 16-byte vector each; a compiler fence between groups keeps only one group's
    // factors live (the query fragments stay in registers).
    f32x4_t kf[4];
    float mt = -INFINITY;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int t0 = 32 * tb + 8 * a + 4 * h32;
      if constexpr (FP8) {
        asm volatile("" ::: "memory");
        kf[a] = *reinterpret_cast<const MLA_LDS f32x4_t*>(ks + t0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 4 * a + j;
        float x = FP8 ? sc[i] * kf[a][j] : sc[i] * scale_log2;
        if (need_mask) x = (tok0 + t0 + j < nvis) ? x : -INFINITY;
        sc[i] = x;
        mt = fmaxf(mt, x);
      }
    }
    mt = fmaxf(mt, shfl_xor_f(mt, 32));
    if (first) st.m = (tb == 0) ? mt : st.m;          // reference from the unit's first block
    st.m_seen = fmaxf(st.m_seen, mt);
    const float base = st.m == -INFINITY ? 0.f : st.m;
    if (mt > base + kRefSlack) *overflow = 1;
    // For each 16-token k-step jj (elements 8jj .. 8jj+7 of this lane) the weights are
    // exponentiated, packed to bf16 and consumed by that step's 16 PV MFMAs right
    // away, so only one step's weights and per-token factors are live at a time.
    // The row sum accumulates the bf16-rounded weights the MFMA actually uses, so the
    // output is an exact convex combination of the V rows: the rounding of a dominant
    // weight then largely cancels instead of scaling the output.
    float lsum = 0.f, lrsum = 0.f;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      bf16x8_t pb;
#pragma unroll
      for (int ah = 0; ah < 2; ++ah) {
        const int a = 2 * jj + ah;
        const int t0 = 32 * tb + 8 * a + 4 * h32;
        f32x4_t vf, ivf;
        if constexpr (FP8) {
          asm volatile("" ::: "memory");
          vf = *reinterpret_cast<const MLA_LDS f32x4_t*>(vs + t0);
          ivf = *reinterpret_cast<const MLA_LDS f32x4_t*>(ivs + t0);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float pr = __builtin_amdgcn_exp2f(sc[4 * a + j] - base);
          const float v = FP8 ? pr * vf[j] : pr;
          const __bf16 r = (__bf16)v;
          pb[4 * ah + j] = r;
          lsum += pr;
          lrsum += FP8 ? (float)r * ivf[j] : (float)r;
        }
      }
      // O^T += V^T . P^T for token step u = 2*tb + jj (tokens 16u .. 16u+15); the two
      // transpose reads of each V^T fragment are issued kPrefV MFMAs ahead.
      const int u = 2 * tb + jj;
      constexpr int kPrefV = 3;
      const uint32_t uofs = (uint32_t)(16 * u * 8 * 16);
      bf16x4_t vlo[kPrefV], vhi[kPrefV];
#pragma unroll
      for (int d = 0; d < kPrefV; ++d) {
        const uint32_t off = vbase[d & 1] + (d >> 1) * kGroupBytes + uofs;
        vlo[d] = lds_read_tr16(pg, off);
        vhi[d] = lds_read_tr16(pg, off + 8 * 8 * 16);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPrefV, 0);         // prologue reads first
#pragma unroll
      for (int fb = 0; fb < 16; ++fb) {
        const bf16x4_t v0 = vlo[fb % kPrefV], v1 = vhi[fb % kPrefV];
        const int nf = fb + kPrefV;
        if (nf < 16) {
          const uint32_t off = vbase[nf & 1] + (nf >> 1) * kGroupBytes + uofs;
          vlo[fb % kPrefV] = lds_read_tr16(pg, off);
          vhi[fb % kPrefV] = lds_read_tr16(pg, off + 8 * 8 * 16);
        }
        const bf16x8_t va = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        st.o[fb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, st.o[fb], 0, 0, 0);
        if (nf < 16) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0); // 2 DS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);             // MFMA
      }
    }
    st.l += lsum;
    st.lr += lrsum;
  }
}

// ---------------------------------------------------------------------------
// Per-unit compute: narrow variant (16 query rows; wave w takes tokens
// 16w..16w+15 of every page; 16x16x32 MFMA for scores, 16x16x16 for PV)
// ---------------------------------------------------------------------------
struct NarrowState {
  f32x4_t o[32];      // O^T: 32 blocks of 16 latent features x 16 rows (lane%16 = row)
  float m, l, lr, m_seen;   // as in WideState
};

template <bool FP8>
__device__ __forceinline__ void narrow_page(const MLA_LDS char* pg, const MLA_LDS float* ks,
                                            const MLA_LDS float* vs, const MLA_LDS float* ivs,
                                            const bf16x8_t (&qf)[18],
                                            NarrowState& st, int tok0, int nvis, bool need_mask,
                                            float scale_log2, int w, int l, bool first,
                                            MLA_LDS int* overflow) {
  const int g = l >> 4, lg = l & 15;
  f32x4_t s = {};
  // K chunk c = 4*kk + g of token 16w + lg: group kk >> 1, in-group chunk 4*(kk & 1) + g
  uint32_t kbase[2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
    kbase[m] = (uint32_t)((16 * w + lg) * 8 + ((4 * m + g) ^ page_swz(lg))) * 16;
#pragma unroll
  for (int kk = 0; kk < 18; ++kk) {
    const bf16x8_t a = lds_read_b128(pg, kbase[kk & 1] + (kk >> 1) * kGroupBytes);
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[kk], s, 0, 0, 0);
  }
  float mt = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = 16 * w + 4 * g + i;
    // fp8: ks[] already holds k_scale * softmax scale * log2(e)
    float x = FP8 ? s[i] * ks[t] : s[i] * scale_log2;
    if (need_mask) x = (tok0 + t < nvis) ? x : -INFINITY;
    s[i] = x;
    mt = fmaxf(mt, x);
  }
  mt = fmaxf(mt, shfl_xor_f(mt, 16));
  mt = fmaxf(mt, shfl_xor_f(mt, 32));
  if (first) st.m = mt;                                // reference from the unit's first page
  st.m_seen = fmaxf(st.m_seen, mt);
  const float base = st.m == -INFINITY ? 0.f : st.m;
  if (mt > base + kRefSlack) *overflow = 1;
  // row sum of the bf16-rounded weights (see wide_page)
  float lsum = 0.f, lrsum = 0.f;
  bf16x4_t pb;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = 16 * w + 4 * g + i;
    const float pr = __builtin_amdgcn_exp2f(s[i] - base);
    const float v = FP8 ? pr * vs[t] : pr;
    const __bf16 r = (__bf16)v;
    pb[i] = r;
    lsum += pr;
    lrsum += FP8 ? (float)r * ivs[t] : (float)r;
  }
  st.l += lsum;
  st.lr += lrsum;
  // V^T transpose reads: token 16w + 4g + (lg >> 2), chunk c = 2*fb + ((lg & 3) >> 1) in
  // group fb >> 2 at in-group chunk 2*(fb & 3) + ((lg & 3) >> 1)
  const int tok = 16 * w + 4 * g + (lg >> 2);
  uint32_t vbase[4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
    vbase[m] = (uint32_t)(tok * 8 + ((2 * m + ((lg & 3) >> 1)) ^ page_swz(tok))) * 16 +
               (uint32_t)(lg & 1) * 8;
#pragma unroll
  for (int fb = 0; fb < 32; ++fb) {
    const bf16x4_t va = lds_read_tr16(pg, vbase[fb & 3] + (fb >> 2) * kGroupBytes);
    st.o[fb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, st.o[fb], 0, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// The persistent decode kernel
// ---------------------------------------------------------------------------
template <bool FP8, bool WIDE>
__global__ __launch_bounds__(256, 1) void decode_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[kLdsBytes];
  MLA_LDS char* smem = (MLA_LDS char*)(smem_raw);
  const int tid = threadIdx.x;
  const int w = wave_id();
  const int l = lane_id();
  const int P = p.hdr[0];
  const int U = p.hdr[1];

  for (int u = blockIdx.x; u < U; u += gridDim.x) {
    int pi, hg;
    unit_to_pair(u, p.n_hg, &pi, &hg);
    if (pi >= P) continue;
    const int4 pr = p.pairs[pi];
    const int b = pr.x, t_begin = pr.z, t_end = pr.w;
    const int4 rq = p.req[b];
    const int nsplit = rq.y, seq = rq.w;
    const int pg0 = t_begin / kPage;
    const int pg1 = t_end > t_begin ? (t_end + kPage - 1) / kPage : pg0;
    const int first_nvis = seq - p.q_len + 1;          // visible tokens of query row 0

    // the row this lane owns in the S^T / O^T accumulators
    const int r = WIDE ? (32 * w + (l & 31)) : (l & 15);
    const int hl = r / p.q_len, tq = r - hl * p.q_len;
    const int head = hg * p.hg_heads + hl;
    const bool row_ok = head < p.N;
    const int nvis = seq - p.q_len + 1 + tq;

    // stage the unit's first page before loading the query fragments
    MLA_LDS char* buf0 = smem + (FP8 ? kFp8Raw0 : 0);
    MLA_LDS char* buf1 = smem + (FP8 ? kFp8Raw1 : kPageBytesBf16);
    PageIds ids;
    load_page_ids(ids, p, b, pg0, pg1, l);
    if (pg1 > pg0) {
      if constexpr (FP8) issue_page_fp8(page_ptr(ids, p, b, pg0, pg1, l, true), buf0, w, l);
      else issue_page_bf16(page_ptr(ids, p, b, pg0, pg1, l, false), buf0, w, l);
    }

    // query fragments (B operand): row r, features 16*kk + 8*(l>>5) (wide) or
    // 32*kk + 8*(l>>4) (narrow)
    constexpr int NQ = WIDE ? 36 : 18;
    bf16x8_t qf[NQ];
    {
      // padding rows (head >= N) load head 0 and are zeroed: no divergent loads
      const uint16_t* qrow = p.q + (int64_t)b * p.q_sb + (int64_t)tq * p.q_st + (int64_t)(row_ok ? head : 0) * p.q_sh;
      const int off = WIDE ? 8 * (l >> 5) : 8 * (l >> 4);
#pragma unroll
      for (int kk = 0; kk < NQ; ++kk) qf[kk] = *reinterpret_cast<const bf16x8_t*>(qrow + (WIDE ? 16 : 32) * kk + off);
      if (!row_ok) {
#pragma unroll
        for (int kk = 0; kk < NQ; ++kk) qf[kk] = bf16x8_t{};
      }
    }

    WideState ws;
    NarrowState ns;
    MLA_LDS int* ovf = reinterpret_cast<MLA_LDS int*>(smem + kLdsFlag);
    float m_restart = -INFINITY;
    for (int attempt = 0; attempt < 2; ++attempt) {
      if constexpr (WIDE) {
#pragma unroll
        for (int i = 0; i < 16; ++i) ws.o[i] = f32x16_t{};
        ws.m = m_restart;
        ws.l = 0.f;
        ws.lr = 0.f;
        ws.m_seen = -INFINITY;
      } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) ns.o[i] = f32x4_t{};
        ns.m = m_restart;
        ns.l = 0.f;
        ns.lr = 0.f;
        ns.m_seen = -INFINITY;
      }
      // reset the flag and make the reset visible before any wave can read it
      // (a unit without pages reads it right after this barrier)
      if (tid == 0) *ovf = 0;
      lds_barrier();
      if (attempt > 0 && pg1 > pg0) {
        load_page_ids(ids, p, b, pg0, pg1, l);
        if constexpr (FP8) issue_page_fp8(page_ptr(ids, p, b, pg0, pg1, l, true), buf0, w, l);
        else issue_page_bf16(page_ptr(ids, p, b, pg0, pg1, l, false), buf0, w, l);
      }

      for (int pg = pg0; pg < pg1; ++pg) {
        const bool odd = ((pg - pg0) & 1) != 0;
        MLA_LDS char* cur = odd ? buf1 : buf0;
        MLA_LDS char* nxt = odd ? buf0 : buf1;
        if (pg + 1 < pg1) {
          if constexpr (FP8) {
            issue_page_fp8(page_ptr(ids, p, b, pg + 1, pg1, l, true), nxt, w, l);
            if (w == 0) wait_vmcnt<10>();
            else wait_vmcnt<9>();
          } else {
            issue_page_bf16(page_ptr(ids, p, b, pg + 1, pg1, l, false), nxt, w, l);
            wait_vmcnt<18>();
          }
        } else {
          wait_vmcnt<0>();
        }
        lds_barrier();
        const int tok0 = pg * kPage;
        const int valid = seq - tok0 < kPage ? seq - tok0 : kPage;
        const MLA_LDS char* page;
        MLA_LDS float* ksc = reinterpret_cast<MLA_LDS float*>(smem + kFp8KScale);
        MLA_LDS float* vsc = reinterpret_cast<MLA_LDS float*>(smem + kFp8VScale);
        MLA_LDS float* ivsc = reinterpret_cast<MLA_LDS float*>(smem + kFp8IVScale);
        if constexpr (FP8) {
          convert_fp8_page(cur, smem + kFp8Conv, ksc, vsc, ivsc, valid, tid, p.scale_log2);
          lds_barrier();
          page = smem + kFp8Conv;
        } else {
          if (valid < kPage) {
            zero_tail_rows(cur, valid, tid);
            lds_barrier();
          }
          page = cur;
        }
        const bool need_mask = tok0 + kPage > first_nvis;
        const bool first = attempt == 0 && pg == pg0;
        if constexpr (WIDE)
          wide_page<FP8>(page, ksc, vsc, ivsc, qf, ws, tok0, nvis, need_mask, p.scale_log2, l, first, ovf);
        else
          narrow_page<FP8>(page, ksc, vsc, ivsc, qf, ns, tok0, nvis, need_mask, p.scale_log2, w, l, first, ovf);
        lds_barrier();
      }
      // every wave reads the flag after the last barrier; the second barrier keeps a
      // fast wave from clearing it (next attempt or unit) before all have read it
      const int redo = *ovf;
      lds_barrier();
      if (redo == 0) break;
      m_restart = WIDE ? ws.m_seen : ns.m_seen;
    }

    // ---- epilogue ----
    const size_t slot = (size_t)pi * p.n_hg + hg;
    if constexpr (WIDE) {
      // Each lane holds O^T for one row (l & 31) and features 32*fb + 8*a + 4*h32 + [0,4).
      // The rows are staged through this wave's own LDS region (rows padded to
      // 1040 B so that 32 lanes writing 32 rows hit distinct banks) and written back
      // row by row, 64 lanes x 16 B = 1 KiB contiguous per store instruction.
      const int h32 = l >> 5;
      const int rl = l & 31;
      const float l_tot = ws.l + shfl_xor_f(ws.l, 32);
      const float lr_tot = ws.lr + shfl_xor_f(ws.lr, 32);
      const float inv = lr_tot > 0.f ? 1.0f / lr_tot : 0.f;
      const float lse_v = l_tot > 0.f ? (ws.m + __builtin_log2f(l_tot)) * kLn2 : -INFINITY;
      constexpr int kRowPad = 1040;
      MLA_LDS char* stage = smem + w * (32 * kRowPad);
      const bool single = nsplit == 1;
      // 32 rows of this wave: row r0 + i maps to (head, q row) like the lanes' own rows
      const int nhalf = single ? 1 : 2;               // bf16: 512 x 2 B per row; fp32: two halves of 256
      for (int hf = 0; hf < nhalf; ++hf) {
        if (single) {
#pragma unroll
          for (int fb = 0; fb < 16; ++fb)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
              const bf16x4_t v = {(__bf16)(ws.o[fb][4 * a] * inv), (__bf16)(ws.o[fb][4 * a + 1] * inv),
                                  (__bf16)(ws.o[fb][4 * a + 2] * inv), (__bf16)(ws.o[fb][4 * a + 3] * inv)};
              *reinterpret_cast<MLA_LDS bf16x4_t*>(stage + rl * kRowPad + (32 * fb + 8 * a + 4 * h32) * 2) = v;
            }
        } else {
#pragma unroll
          for (int fb = 0; fb < 16; ++fb) {
            if ((fb >> 3) != hf) continue;
#pragma unroll
            for (int a = 0; a < 4; ++a) {
              const f32x4_t v = {ws.o[fb][4 * a] * inv, ws.o[fb][4 * a + 1] * inv, ws.o[fb][4 * a + 2] * inv,
                                 ws.o[fb][4 * a + 3] * inv};
              *reinterpret_cast<MLA_LDS f32x4_t*>(stage + rl * kRowPad + (32 * (fb & 7) + 8 * a + 4 * h32) * 4) = v;
            }
          }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's stage is written
        for (int i = 0; i < 32; ++i) {
          const int rr = 32 * w + i;
          const int hl_i = rr / p.q_len, tq_i = rr - hl_i * p.q_len;
          const int head_i = hg * p.hg_heads + hl_i;
          if (head_i >= p.N) continue;                        // uniform
          const u32x4_t v = *reinterpret_cast<const MLA_LDS u32x4_t*>(stage + i * kRowPad + l * 16);
          if (single) {
            uint16_t* orow = p.out + (int64_t)b * p.o_sb + (int64_t)tq_i * p.o_st + (int64_t)head_i * p.o_sh;
            *reinterpret_cast<u32x4_t*>(orow + 8 * l) = v;
          } else {
            float* prow = p.part_o + (slot * p.m_wg + rr) * kLatent + 256 * hf;
            *reinterpret_cast<u32x4_t*>(prow + 4 * l) = v;
          }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // reads done before the stage is reused
      }
      if (row_ok && h32 == 0) {
        if (single) p.lse[((int64_t)b * p.q_len + tq) * p.N + head] = lse_v;
        else p.part_lse[slot * p.m_wg + r] = lse_v;
      }
      lds_barrier();                                          // stages free before the next unit's DMA
    } else {
      // combine the four token-slices of the waves through LDS
      float l_w = ns.l + shfl_xor_f(ns.l, 16);
      l_w += shfl_xor_f(l_w, 32);
      float lr_w = ns.lr + shfl_xor_f(ns.lr, 16);
      lr_w += shfl_xor_f(lr_w, 32);
      MLA_LDS float* obuf = reinterpret_cast<MLA_LDS float*>(smem);
      MLA_LDS float* stat = reinterpret_cast<MLA_LDS float*>(smem + 4 * 16 * kLatent * 4);
      const int g = l >> 4;
#pragma unroll
      for (int fb = 0; fb < 32; ++fb)
        *reinterpret_cast<MLA_LDS f32x4_t*>(obuf + (w * 16 + r) * kLatent + 16 * fb + 4 * g) = ns.o[fb];
      if (l < 16) {
        stat[(w * 16 + r) * 4] = ns.m;
        stat[(w * 16 + r) * 4 + 1] = l_w;
        stat[(w * 16 + r) * 4 + 2] = lr_w;
      }
      lds_barrier();
      const int rr = tid >> 4;                 // row 0..15
      const int fp = tid & 15;                 // features 64*j + 4*fp + [0,4), j = 0..7:
                                               // 16 lanes of a row store 256 contiguous bytes
      float mw[4], lw[4], lrw[4];
      float M = -INFINITY;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        mw[k] = stat[(k * 16 + rr) * 4];
        lw[k] = stat[(k * 16 + rr) * 4 + 1];
        lrw[k] = stat[(k * 16 + rr) * 4 + 2];
        M = fmaxf(M, mw[k]);
      }
      const float Mb = M == -INFINITY ? 0.f : M;
      float wgt[4], L = 0.f, LR = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        wgt[k] = __builtin_amdgcn_exp2f(mw[k] - Mb);
        L += wgt[k] * lw[k];
        LR += wgt[k] * lrw[k];
      }
      const float inv = LR > 0.f ? 1.0f / LR : 0.f;
      const float lse_v = L > 0.f ? (Mb + __builtin_log2f(L)) * kLn2 : -INFINITY;
      const int rhl = rr / p.q_len, rtq = rr - rhl * p.q_len;
      const int rhead = hg * p.hg_heads + rhl;
      if (rhead < p.N) {
        f32x4_t acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = f32x4_t{};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const MLA_LDS float* src = obuf + (k * 16 + rr) * kLatent + 4 * fp;
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[j] += wgt[k] * *reinterpret_cast<const MLA_LDS f32x4_t*>(src + 64 * j);
        }
        if (nsplit == 1) {
          uint16_t* orow = p.out + (int64_t)b * p.o_sb + (int64_t)rtq * p.o_st + (int64_t)rhead * p.o_sh + 4 * fp;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const bf16x4_t v = {(__bf16)(acc[j][0] * inv), (__bf16)(acc[j][1] * inv), (__bf16)(acc[j][2] * inv),
                                (__bf16)(acc[j][3] * inv)};
            *reinterpret_cast<bf16x4_t*>(orow + 64 * j) = v;
          }
          if (fp == 0) p.lse[((int64_t)b * p.q_len + rtq) * p.N + rhead] = lse_v;
        } else {
          float* prow = p.part_o + (slot * p.m_wg + rr) * kLatent + 4 * fp;
#pragma unroll
          for (int j = 0; j < 8; ++j) *reinterpret_cast<f32x4_t*>(prow + 64 * j) = acc[j] * inv;
          if (fp == 0) p.part_lse[slot * p.m_wg + rr] = lse_v;
        }
      }
      lds_barrier();
    }
  }
}

// ---------------------------------------------------------------------------
// Split merge: grid = (B * n_hg, ceil(m_wg / 16)); each wave merges 4 rows, each
// lane 8 of the 512 latent features.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void merge_kernel(DecodeParams p) {
  // grid = (B * n_hg, ceil(m_wg / 16)): each wave merges 4 rows; lane s < nsplit fetches
  // split s's lse, so the max and the weights take one load and a wave reduction; each
  // lane then accumulates 8 of the 512 features over the splits, 4 splits' loads in flight.
  const int b = blockIdx.x / p.n_hg;
  const int hg = blockIdx.x - b * p.n_hg;
  const int4 rq = p.req[b];
  const int first = rq.x, nsplit = rq.y;
  if (nsplit <= 1) return;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  for (int j = 0; j < 4; ++j) {
    const int r = blockIdx.y * 16 + w * 4 + j;
    if (r >= p.m_wg) break;
    const int hl = r / p.q_len, tq = r - hl * p.q_len;
    const int head = hg * p.hg_heads + hl;
    if (head >= p.N) continue;
    float M = -INFINITY;
    for (int s0 = 0; s0 < nsplit; s0 += 64) {
      const int s = s0 + l;
      const float ls = s < nsplit ? p.part_lse[((size_t)(first + s) * p.n_hg + hg) * p.m_wg + r] : -INFINITY;
      M = fmaxf(M, ls);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, shfl_xor_f(M, m));
    const float Mb = M == -INFINITY ? 0.f : M;
    f32x4_t a0 = {}, a1 = {};
    float wsum = 0.f;
    int s = 0;
    for (; s + 4 <= nsplit; s += 4) {
      f32x4_t v[4][2];
      float wt[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const size_t slot = (size_t)(first + s + k) * p.n_hg + hg;
        const f32x4_t* src = reinterpret_cast<const f32x4_t*>(p.part_o + (slot * p.m_wg + r) * kLatent + 8 * l);
        v[k][0] = src[0];
        v[k][1] = src[1];
        const float ls = p.part_lse[slot * p.m_wg + r];
        wt[k] = ls == -INFINITY ? 0.f : __expf(ls - Mb);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        wsum += wt[k];
        a0 += wt[k] * v[k][0];
        a1 += wt[k] * v[k][1];
      }
    }
    for (; s < nsplit; ++s) {
      const size_t slot = (size_t)(first + s) * p.n_hg + hg;
      const f32x4_t* src = reinterpret_cast<const f32x4_t*>(p.part_o + (slot * p.m_wg + r) * kLatent + 8 * l);
      const float ls = p.part_lse[slot * p.m_wg + r];
      const float wt = ls == -INFINITY ? 0.f : __expf(ls - Mb);
      wsum += wt;
      a0 += wt * src[0];
      a1 += wt * src[1];
    }
    const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
    uint16_t* orow = p.out + (int64_t)b * p.o_sb + (int64_t)tq * p.o_st + (int64_t)head * p.o_sh + 8 * l;
    const bf16x8_t v = {(__bf16)(a0[0] * inv), (__bf16)(a0[1] * inv), (__bf16)(a0[2] * inv),
                        (__bf16)(a0[3] * inv), (__bf16)(a1[0] * inv), (__bf16)(a1[1] * inv),
                        (__bf16)(a1[2] * inv), (__bf16)(a1[3] * inv)};
    *reinterpret_cast<bf16x8_t*>(orow) = v;
    if (l == 0) p.lse[((int64_t)b * p.q_len + tq) * p.N + head] = wsum > 0.f ? Mb + __logf(wsum) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
struct Shape {
  bool wide;
  int m_wg, hg_heads, n_hg, max_pairs;
};

inline bool decode_shape(int32_t B, int32_t q_len, int32_t N, int32_t num_splits, Shape* s) {
  if (B < 1 || (q_len != 1 && q_len != 2) || N < 1 || N > MLA_MAX_HEADS) return false;
  if (num_splits < 0 || num_splits > 4096) return false;
  s->wide = q_len * N > 16;
  s->m_wg = s->wide ? 128 : 16;
  s->hg_heads = s->m_wg / q_len;
  s->n_hg = (N + s->hg_heads - 1) / s->hg_heads;
  int64_t mp;
  if (num_splits == 0) mp = (int64_t)B + MLA_AUTO_MAX_EXTRA_PAIRS;
  else mp = (int64_t)B * num_splits;
  mp += 8;
  if (mp > (1 << 24)) return false;
  s->max_pairs = (int)mp;
  return true;
}

struct WsLayout {
  size_t hdr, req, pairs, part_lse, part_o, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline WsLayout ws_layout(int32_t B, const Shape& s) {
  WsLayout w;
  size_t off = 0;
  w.hdr = off;
  off = align256(off + 16 * sizeof(int32_t));
  w.req = off;
  off = align256(off + (size_t)B * sizeof(int4));
  w.pairs = off;
  off = align256(off + (size_t)s.max_pairs * sizeof(int4));
  const size_t rows = (size_t)s.max_pairs * s.n_hg * s.m_wg;
  w.part_lse = off;
  off = align256(off + rows * sizeof(float));
  w.part_o = off;
  off = align256(off + rows * kLatent * sizeof(float));
  w.total = off;
  return w;
}

}  // namespace mla

extern "C" size_t mla_decode_workspace_size(int32_t B, int32_t q_len, int32_t N, int32_t num_splits) {
  mla::Shape s;
  if (!mla::decode_shape(B, q_len, N, num_splits, &s)) return 0;
  return mla::ws_layout(B, s).total;
}

extern "C" mla_status_t mla_decode(const void* q, int64_t q_stride_b, int64_t q_stride_t,
                                   int64_t q_stride_h, const void* kv_cache, int32_t kv_dtype,
                                   int64_t num_pages, const int32_t* block_table, int64_t bt_stride_b,
                                   int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t B,
                                   int32_t q_len, int32_t N, float softmax_scale, int32_t num_splits,
                                   void* workspace, size_t workspace_bytes, void* out,
                                   int64_t o_stride_b, int64_t o_stride_t, int64_t o_stride_h,
                                   float* lse, void* stream) {
  using namespace mla;
  if (kv_dtype != MLA_KV_BF16 && kv_dtype != MLA_KV_FP8_E4M3) return MLA_ERR_DTYPE;
  Shape s;
  if (!decode_shape(B, q_len, N, num_splits, &s)) return MLA_ERR_SHAPE;
  if (num_pages < 1 || max_pages_per_seq < 1 || bt_stride_b < max_pages_per_seq) return MLA_ERR_SHAPE;
  if (!(softmax_scale > 0.f) || !__builtin_isfinite(softmax_scale)) return MLA_ERR_SHAPE;
  if (!q || !kv_cache || !block_table || !seq_lens || !out || !lse) return MLA_ERR_NULL;
  if (!workspace) return MLA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(kv_cache) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 || !mult8(q_stride_b) ||
      !mult8(q_stride_t) || !mult8(q_stride_h) || !mult8(o_stride_b) || !mult8(o_stride_t) ||
      !mult8(o_stride_h) || (reinterpret_cast<uintptr_t>(block_table) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3u) != 0 || (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
    return MLA_ERR_ALIGN;
  const WsLayout wl = ws_layout(B, s);
  if (workspace_bytes < wl.total) return MLA_ERR_WORKSPACE;
  DeviceInfo di;
  mla_status_t st = device_info(&di);
  if (st != MLA_OK) return st;

  char* ws = static_cast<char*>(workspace);
  DecodeParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.q_sb = q_stride_b;
  p.q_st = q_stride_t;
  p.q_sh = q_stride_h;
  p.kv = static_cast<const char*>(kv_cache);
  p.num_pages = num_pages;
  p.block_table = block_table;
  p.bt_sb = bt_stride_b;
  p.max_pages = max_pages_per_seq;
  p.seq_lens = seq_lens;
  p.B = B;
  p.q_len = q_len;
  p.N = N;
  p.n_hg = s.n_hg;
  p.m_wg = s.m_wg;
  p.hg_heads = s.hg_heads;
  p.scale_log2 = softmax_scale * kLog2e;
  p.out = static_cast<uint16_t*>(out);
  p.o_sb = o_stride_b;
  p.o_st = o_stride_t;
  p.o_sh = o_stride_h;
  p.lse = lse;
  p.hdr = reinterpret_cast<int32_t*>(ws + wl.hdr);
  p.req = reinterpret_cast<int4*>(ws + wl.req);
  p.pairs = reinterpret_cast<int4*>(ws + wl.pairs);
  p.part_lse = reinterpret_cast<float*>(ws + wl.part_lse);
  p.part_o = reinterpret_cast<float*>(ws + wl.part_o);
  p.max_pairs = s.max_pairs;
  p.num_splits = num_splits;
  // automatic plan: about one work unit per CU for the wide kernel (one
  // 256-thread workgroup fills a CU) and four per CU for the short narrow units
  int target_units = s.wide ? di.cu_count : 4 * di.cu_count;
  int tp = target_units / s.n_hg;
  if (tp < 1) tp = 1;
  if (tp > MLA_AUTO_MAX_EXTRA_PAIRS) tp = MLA_AUTO_MAX_EXTRA_PAIRS;
  p.target_pairs = tp;

  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, hs, p);
  if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;

  const int64_t max_units = s.n_hg == 1 ? s.max_pairs : ((s.max_pairs + 7) / 8) * 8 * (int64_t)s.n_hg;
  int64_t grid = (int64_t)di.cu_count;
  grid = (grid + 7) / 8 * 8;
  if (grid > max_units) grid = (max_units + 7) / 8 * 8;
  if (grid < 8) grid = 8;
  if (kv_dtype == MLA_KV_BF16) {
    if (s.wide) hipLaunchKernelGGL((decode_kernel<false, true>), dim3((unsigned)grid), dim3(256), 0, hs, p);
    else hipLaunchKernelGGL((decode_kernel<false, false>), dim3((unsigned)grid), dim3(256), 0, hs, p);
  } else {
    if (s.wide) hipLaunchKernelGGL((decode_kernel<true, true>), dim3((unsigned)grid), dim3(256), 0, hs, p);
    else hipLaunchKernelGGL((decode_kernel<true, false>), dim3((unsigned)grid), dim3(256), 0, hs, p);
  }
  if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;
  if (num_splits != 1) {
    dim3 mg((unsigned)(B * s.n_hg), (unsigned)((s.m_wg + 15) / 16));
    hipLaunchKernelGGL(merge_kernel, mg, dim3(256), 0, hs, p);
  }
  return launch_status();
}
