// Prefill of new tokens, the compute-friendly MLA path: multi-head attention with
// 192-wide keys [k_nope[s,h] | k_pe[s]] (the one rope key shared by every head) and
// 128-wide values, ragged causal requests, output plus natural-log LSE so that a
// context part can be merged in with mla_merge_attn_states.
// Source: "vLLM 源码完全拆解(三十七):MLA 注意力后端", §两套算法 (compute-friendly form
// for prefill, softmax scale 1/sqrt(192)) and §Prefill (run_prefill_new_tokens: keys
// and values from kv_b_proj, k_pe broadcast over heads, causal over the new tokens
// after the request's context).
//
// One workgroup per (256 query rows, head, request): eight waves, two per SIMD, each
// owning 32 query rows.  The scores use 32x32x16 bf16 MFMAs with the query rows in
// registers as the B operand: they come out as S^T (keys x queries), each lane holding
// 32 keys of one query and lane l ^ 32 the other 32, one permlane32 swap away.  Keys
// stream in blocks of 64, copied straight from global memory into LDS
// (global_load_lds) through a ring of three buffers, so that a block's copy is issued
// two blocks ahead of its use; each buffer holds three XOR-swizzled row-major regions,
// k_nope, k_pe and values, whose swizzles keep the MFMA operand reads free of bank
// conflicts.  The values are read with ds_read_b64_tr_b16 as the A operand of
// O^T = V^T P^T, the lane's own probabilities being the B operand: both take the keys
// in the same permuted order (k index 8h + e of a 16-key step is key 8(e/4) + 4h + e%4
// of the step, h the lane's half).  The softmax keeps a fixed reference maximum per row,
// the first block's, so that the output accumulators are never rescaled in the key
// loop; a row whose scores later rise more than 2^64 above it (a probability the fp32
// accumulators still hold) sends the workgroup through a second pass from the largest
// maxima seen.  Workgroups are numbered so that the ones sharing a (request, head), and
// with it its keys and values, run on the same XCD (one L2), the longest causal tiles
// first.
#include "mla_common.h"
#include "mla_host.h"

namespace mla {

struct PrefillParams {
  const uint16_t* q;       // [T, N, 192]
  const uint16_t* kn;      // [S, N, 128]
  const uint16_t* kp;      // [S, 64]
  const uint16_t* v;       // [S, N, 128]
  const int32_t* cu_q;     // [B + 1]
  const int32_t* cu_k;     // [B + 1]
  uint16_t* out;           // [T, N, 128]
  float* lse;              // [T, N]
  int64_t q_st, q_sh, kn_st, kn_sh, kp_st, v_st, v_sh, o_st, o_sh;
  int64_t T, S;
  int32_t N, causal;
  float scale_log2;        // softmax scale times log2(e)
};

constexpr int kPW = 8;               // waves per workgroup, two per SIMD
constexpr int kPQ = kPW * 32;        // query rows per workgroup
constexpr int kPK = 64;              // keys per block
constexpr int kRing = 4;             // LDS buffers: blocks j + 2, j + 3 are copied while j, j + 1 are used
// one LDS buffer: k_nope [64][256 B], k_pe [64][128 B], values [64][256 B], each row's
// 16-byte chunks XOR-swizzled (chunk c of row r at c ^ (r & 15), c ^ ((r >> 1) & 7) and
// c ^ 4(r & 3) respectively)
constexpr int kKnBytes = kPK * 256;
constexpr int kKpBytes = kPK * 128;
constexpr int kVBytes = kPK * 256;
constexpr int kBufBytes = kKnBytes + kKpBytes + kVBytes;   // 40 KiB
constexpr float kSlack = 64.f;       // log2 of the largest probability a fixed reference allows

// DMA of one block: 40 instructions of 64 x 16 B (16 k_nope, 8 k_pe, 16 values); wave w
// issues k_nope and value instructions i = 8j + w (j = 0, 1) and k_pe instruction w,
// instruction i of a region covering its 16-byte positions 64i .. 64i + 63.  In a whole
// block the swizzle of a lane's row does not depend on j, so instruction j differs only
// by 32 rows, which go into the scalar base; the lane keeps one offset per region.  A
// request's last block clamps the rows to its last key (rows past it are masked or
// multiplied by zero) and takes per-instruction offsets.
struct PrefillDma {
  uint32_t kn, kp, v;
};

__device__ __forceinline__ PrefillDma prefill_dma_offsets(const PrefillParams& p, int w, int L) {
  PrefillDma d;
  const int r = 4 * w + (L >> 4), rp = 8 * w + (L >> 3);
  d.kn = (uint32_t)(r * p.kn_st * 2 + (((L & 15) ^ (r & 15)) * 16));
  d.v = (uint32_t)(r * p.v_st * 2 + (((L & 15) ^ (4 * (r & 3))) * 16));
  d.kp = (uint32_t)(rp * p.kp_st * 2 + (((L & 7) ^ ((rp >> 1) & 7)) * 16));
  return d;
}

__device__ __forceinline__ void prefill_issue_full(const PrefillParams& p, const PrefillDma& d, const char* kn,
                                                   const char* kp, const char* v, uint32_t lds) {
  dma_16B<0, 0>(kn, d.kn, lds);
  dma_16B<0, 8192>(kn + (int64_t)32 * p.kn_st * 2, d.kn, lds);
  dma_16B<0, kKnBytes>(kp, d.kp, lds);
  dma_16B<0, kKnBytes + kKpBytes>(v, d.v, lds);
  dma_16B<0, kKnBytes + kKpBytes + 8192>(v + (int64_t)32 * p.v_st * 2, d.v, lds);
}

__device__ __forceinline__ void prefill_issue_tail(const PrefillParams& p, int w, int L, int n, const char* kn,
                                                   const char* kp, const char* v, uint32_t lds) {
  const int last = n - 1;
  auto kn_off = [&](int j) {
    const int r = 32 * j + 4 * w + (L >> 4);
    return (uint32_t)(min(r, last) * p.kn_st * 2 + (((L & 15) ^ (r & 15)) * 16));
  };
  auto v_off = [&](int j) {
    const int r = 32 * j + 4 * w + (L >> 4);
    return (uint32_t)(min(r, last) * p.v_st * 2 + (((L & 15) ^ (4 * (r & 3))) * 16));
  };
  const int rp = 8 * w + (L >> 3);
  const uint32_t kp_off = (uint32_t)(min(rp, last) * p.kp_st * 2 + (((L & 7) ^ ((rp >> 1) & 7)) * 16));
  dma_16B<0, 0>(kn, kn_off(0), lds);
  dma_16B<0, 8192>(kn, kn_off(1), lds);
  dma_16B<0, kKnBytes>(kp, kp_off, lds);
  dma_16B<0, kKnBytes + kKpBytes>(v, v_off(0), lds);
  dma_16B<0, kKnBytes + kKpBytes + 8192>(v, v_off(1), lds);
}

__device__ __forceinline__ const char* uniform_ptr(const void* ptr) {
  const uint64_t u = (uint64_t)(uintptr_t)ptr;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<const char*>((uintptr_t)(((uint64_t)hi << 32) | lo));
}

__global__ __launch_bounds__(kPW * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_mha_kernel(
    PrefillParams p, int32_t q_tiles) {
  __shared__ __attribute__((aligned(1024))) char smem[kRing * kBufBytes];

  // work item of this workgroup: workgroups L = 8i + x run on XCD x, so XCD x gets the
  // contiguous item range starting at x * (n / 8) + min(x, n % 8)
  const uint32_t n_items = gridDim.x, L = blockIdx.x;
  const uint32_t xcd = L & 7u, per = n_items >> 3, rem = n_items & 7u;
  const uint32_t item = xcd * per + min(xcd, rem) + (L >> 3);
  const int qt = q_tiles - 1 - (int)(item % (uint32_t)q_tiles);
  const int h = (int)((item / (uint32_t)q_tiles) % (uint32_t)p.N);
  const int b = (int)(item / ((uint32_t)q_tiles * (uint32_t)p.N));

  const int64_t q0 = min<int64_t>(max<int64_t>(p.cu_q[b], 0), p.T);
  const int64_t q1 = min<int64_t>(max<int64_t>(p.cu_q[b + 1], q0), p.T);
  const int64_t k0 = min<int64_t>(max<int64_t>(p.cu_k[b], 0), p.S);
  const int64_t k1 = min<int64_t>(max<int64_t>(p.cu_k[b + 1], k0), p.S);
  const int qlen = (int)min<int64_t>(q1 - q0, 0x7fffffff), klen = (int)min<int64_t>(k1 - k0, 0x7fffffff);
  const int qb = qt * kPQ;
  if (qb >= qlen) return;
  const int w = wave_id(), l = threadIdx.x & 63, hf = l >> 5, l32 = l & 31;
  const int g = l >> 4, lg = l & 15;
  const int ctx = klen - qlen;
  auto vis = [&](int row) { return p.causal ? max(0, min(klen, ctx + row + 1)) : klen; };

  // keys the workgroup needs; this wave's rows, the keys its first and last rows see,
  // and this lane's query (the score column) and its keys
  const int kend = vis(min(qb + kPQ, qlen) - 1);
  // waves w and w + 4 share a SIMD: tiles w and 7 - w, so that every SIMD holds one
  // short and one long causal tile
  const int row0 = qb + 32 * (w < 4 ? w : 11 - w);
  const int kend_w = row0 < qlen ? vis(min(row0 + 32, qlen) - 1) : 0;
  const int nvis_lo = vis(row0);
  const int qi = row0 + l32;
  const bool q_ok = qi < qlen;
  const int nvis = vis(qi);

  // query fragments: B operand, lane = query column, 8 consecutive features per k step
  bf16x8_t qf[12];
  {
    const uint16_t* qrow = p.q + (q0 + (q_ok ? qi : 0)) * p.q_st + (int64_t)h * p.q_sh + 8 * hf;
#pragma unroll
    for (int kk = 0; kk < 12; ++kk) qf[kk] = *reinterpret_cast<const bf16x8_t*>(qrow + 16 * kk);
    // retire the query loads here: the compiler cannot see the copies' own waits in the
    // key loop, and would otherwise wait there on counts that include the copies of the
    // blocks in flight
#pragma unroll
    for (int kk = 0; kk < 12; ++kk) asm volatile("" : "+v"(qf[kk]));
  }

  // operand read offsets in a buffer: k_nope rows l32 (+32 kt) for k steps 0..7, k_pe
  // for steps 8..11, and the value transpose reads (rows 4(g>>1) + (lg>>2) of a 16-key
  // step, 4 columns at 16(g&1) + 4(lg&3) of a 32-feature tile); (2kk + hf) ^ x is
  // 2kk ^ (hf ^ x), so one base per region takes the step or tile XORed in
  const uint32_t a_kn = (uint32_t)(l32 * 256 + 16 * (hf ^ (l & 15)));
  const uint32_t a_kp = (uint32_t)(kKnBytes + l32 * 128 + 16 * (hf ^ ((l32 >> 1) & 7)));
  const uint32_t a_v = (uint32_t)(kKnBytes + kKpBytes + (4 * (g >> 1) + (lg >> 2)) * 256 + 64 * (lg >> 2) +
                                  16 * (2 * (g & 1) + ((lg & 3) >> 1)) + 8 * (lg & 1));

  const PrefillDma dma = prefill_dma_offsets(p, w, l);
  const char* kn_base = uniform_ptr(p.kn + k0 * p.kn_st + (int64_t)h * p.kn_sh);
  const char* kp_base = uniform_ptr(p.kp + k0 * p.kp_st);
  const char* v_base = uniform_ptr(p.v + k0 * p.v_st + (int64_t)h * p.v_sh);
  const uint32_t lds0 = lds_addr((MLA_LDS char*)smem) + 1024u * (uint32_t)w;
  auto issue = [&](int blk) {
    const int kb = blk * kPK;
    const char* kn = kn_base + (int64_t)kb * p.kn_st * 2;
    const char* kp = kp_base + (int64_t)kb * p.kp_st * 2;
    const char* v = v_base + (int64_t)kb * p.v_st * 2;
    const uint32_t dst = lds0 + (uint32_t)((blk % kRing) * kBufBytes);
    if (kb + kPK <= klen) prefill_issue_full(p, dma, kn, kp, v, dst);
    else prefill_issue_tail(p, w, l, klen - kb, kn, kp, v, dst);
  };

  const int nblk = (kend + kPK - 1) / kPK;
  const int nblk_w = (kend_w + kPK - 1) / kPK;
  float m_ref = -INFINITY, m_seen = -INFINITY, lsum = 0.f;
  f32x16_t o[4];
  // one block's scores, softmax and PV (the block is in the ring; this wave has keys in it)
  bool ovf = false;
  auto block = [&](int j) {
    const MLA_LDS char* buf = (MLA_LDS char*)smem + (j % kRing) * kBufBytes;
    const int kb = j * kPK;
    // S^T = K Q^T for two 32-key tiles.  The score MFMAs run at raised wave priority,
    // the softmax and PV at the base one: of the two waves on a SIMD, the one starting
    // its scores issues first and the other's softmax and PV fill its MFMA latency
    // (raising PV's priority too measured 5 % slower).
    __builtin_amdgcn_s_setprio(1);
    f32x16_t s[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
    for (int kk = 0; kk < 12; ++kk) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const uint32_t off = kk < 8 ? (a_kn ^ (uint32_t)(32 * kk)) + kt * 32 * 256
                                    : (a_kp ^ (uint32_t)(32 * (kk - 8))) + kt * 32 * 128;
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read_b128(buf, off), qf[kk], s[kt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // s[kt][r] = score of key kb + 32kt + 8(r/4) + 4hf + r%4 for this lane's query
    if (kb + kPK > nvis_lo) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb + 32 * kt + 8 * (r >> 2) + 4 * hf + (r & 3);
          if (key >= nvis) s[kt][r] = -INFINITY;
        }
    }
    float bmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) bmax = fmaxf(bmax, s[kt][r]);
    bmax = max_xor32(bmax) * p.scale_log2;
    // a row without a reference takes this block's maximum (its output and sum are
    // still zero); one far above the reference flags the workgroup
    m_seen = fmaxf(m_seen, bmax);
    if (m_ref == -INFINITY) m_ref = bmax;
    ovf = ovf || bmax > m_ref + kSlack;
    const float mm = m_ref == -INFINITY ? 0.f : m_ref;
    bf16x8_t pb[4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = __builtin_amdgcn_exp2f(fmaf(s[kt][r], p.scale_log2, -mm));
        pb[2 * kt + (r >> 3)][r & 7] = (__bf16)pr;
        lsum += pr;
      }
    // O^T += V^T P^T over four 16-key steps
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int ft = 0; ft < 4; ++ft) {
        const uint32_t off = (a_v ^ (uint32_t)(64 * ft)) + (uint32_t)((32 * (st >> 1) + 16 * (st & 1)) * 256);
        const bf16x4_t lo = lds_read_tr16(buf, off);
        const bf16x4_t hi = lds_read_tr16(buf, off + 8 * 256);
        const bf16x8_t a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[ft] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[st], o[ft], 0, 0, 0);
      }
    }
  };

  for (int pass = 0; pass < 2; ++pass) {
    ovf = false;
    lsum = 0.f;
#pragma unroll
    for (int ft = 0; ft < 4; ++ft) o[ft] = f32x16_t{};
    if (nblk > 0) issue(0);
    if (nblk > 1) issue(1);
    // blocks in pairs: the barrier before a pair makes both its blocks (this wave waited
    // for its own copies of them) visible and retires the previous pair, whose buffers
    // the next pair's copies then take
    for (int j = 0; j < nblk; j += 2) {
      wait_vmcnt<0>();
      lds_barrier();
      if (j + 2 < nblk) issue(j + 2);
      if (j + 3 < nblk) issue(j + 3);
      if (j < nblk_w) block(j);
      if (j + 1 < nblk_w) block(j + 1);
    }
    __builtin_amdgcn_s_setprio(0);
    // a row over its reference anywhere in the workgroup: every wave runs again with
    // the largest maxima seen (the second pass cannot exceed them).  The vote goes
    // through the first word of buffer 0, idle between passes.
    if (pass == 0) {
      volatile MLA_LDS int* redo_flag = reinterpret_cast<volatile MLA_LDS int*>((MLA_LDS char*)smem);
      lds_barrier();                                   // every wave is done with the ring
      if (threadIdx.x == 0) *redo_flag = 0;
      lds_barrier();
      if (__any(ovf) && l == 0) *redo_flag = 1;
      lds_barrier();
      const int redo = *redo_flag;
      lds_barrier();                                   // the flag is read before the ring is reused
      if (redo == 0) break;
      m_ref = m_seen;
    }
  }

  // o[ft][r] = O[query l32][feature 32ft + 8(r/4) + 4hf + r%4]
  const float tot = sum_xor32(lsum);
  if (q_ok) {
    const float inv = tot > 0.f ? 1.0f / tot : 0.f;
    uint16_t* orow = p.out + (q0 + qi) * p.o_st + (int64_t)h * p.o_sh + 4 * hf;
#pragma unroll
    for (int ft = 0; ft < 4; ++ft)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const bf16x4_t v4 = {(__bf16)(o[ft][4 * rb] * inv), (__bf16)(o[ft][4 * rb + 1] * inv),
                             (__bf16)(o[ft][4 * rb + 2] * inv), (__bf16)(o[ft][4 * rb + 3] * inv)};
        *reinterpret_cast<bf16x4_t*>(orow + 32 * ft + 8 * rb) = v4;
      }
    if (hf == 0) p.lse[(q0 + qi) * p.N + h] = tot > 0.f ? (m_ref + __log2f(tot)) * 0.6931471805599453f : -INFINITY;
  }
}

}  // namespace mla

extern "C" mla_status_t mla_prefill_mha(const void* q, int64_t q_stride_t, int64_t q_stride_h, const void* k_nope,
                                        int64_t kn_stride_t, int64_t kn_stride_h, const void* k_pe,
                                        int64_t kp_stride_t, const void* v, int64_t v_stride_t, int64_t v_stride_h,
                                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t B,
                                        int64_t T, int64_t S, int32_t N, int32_t max_q_len, int32_t causal,
                                        float softmax_scale, void* out, int64_t o_stride_t, int64_t o_stride_h,
                                        float* lse, void* stream) {
  using namespace mla;
  if (B < 0 || B > 65535 || T < 0 || S < 0 || N < 1 || N > MLA_MAX_HEADS || max_q_len < 0) return MLA_ERR_SHAPE;
  if (B == 0 || T == 0 || max_q_len == 0) return MLA_OK;
  if (T > 0x7fffffff || S > 0x7fffffff) return MLA_ERR_SHAPE;
  if (!q || !k_nope || !k_pe || !v || !cu_seqlens_q || !cu_seqlens_k || !out || !lse) return MLA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_nope) || !aligned16(k_pe) || !aligned16(v) || !aligned16(out) ||
      !mult8(q_stride_t) || !mult8(q_stride_h) || !mult8(kn_stride_t) || !mult8(kn_stride_h) ||
      !mult8(kp_stride_t) || !mult8(v_stride_t) || !mult8(v_stride_h) || !mult8(o_stride_t) || !mult8(o_stride_h) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u) || (reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) ||
      (reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3u))
    return MLA_ERR_ALIGN;
  DeviceInfo di;
  mla_status_t st = device_info(&di);
  if (st != MLA_OK) return st;
  PrefillParams p;
  p.q = (const uint16_t*)q;
  p.kn = (const uint16_t*)k_nope;
  p.kp = (const uint16_t*)k_pe;
  p.v = (const uint16_t*)v;
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.out = (uint16_t*)out;
  p.lse = lse;
  p.q_st = q_stride_t; p.q_sh = q_stride_h;
  p.kn_st = kn_stride_t; p.kn_sh = kn_stride_h;
  p.kp_st = kp_stride_t;
  p.v_st = v_stride_t; p.v_sh = v_stride_h;
  p.o_st = o_stride_t; p.o_sh = o_stride_h;
  p.T = T; p.S = S; p.N = N; p.causal = causal ? 1 : 0;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  // a thread's offsets into a 64-key block are 32-bit
  if (kn_stride_t > (1 << 24) || kp_stride_t > (1 << 24) || v_stride_t > (1 << 24) || kn_stride_t < 0 ||
      kp_stride_t < 0 || v_stride_t < 0)
    return MLA_ERR_SHAPE;
  const int32_t q_tiles = (max_q_len + kPQ - 1) / kPQ;
  const int64_t items = (int64_t)q_tiles * N * B;
  if (items > 0x7fffffff) return MLA_ERR_SHAPE;
  hipLaunchKernelGGL(prefill_mha_kernel, dim3((unsigned)items), dim3(kPW * 64), 0,
                     reinterpret_cast<hipStream_t>(stream), p, q_tiles);
  return launch_status();
}

// ---------------------------------------------------------------------------
// Chunked context of a prefill batch ([vLLM-MLA] §Prefill): the row budget of the
// gather workspace and the chunk plan, host arithmetic only.  Each chunk is gathered
// (mla_gather_cache), up-projected (mla_kv_b_proj), attended by the new tokens
// (mla_prefill_mha, not causal: the whole context precedes them) and merged into the
// running state (mla_merge_attn_states), so that at most the row budget of latents is
// up-projected at a time.
// ---------------------------------------------------------------------------
extern "C" int64_t mla_prefill_workspace_rows(int64_t max_model_len, int64_t max_num_seqs, int32_t page_tokens) {
  if (max_model_len < 1 || max_num_seqs < 1 || page_tokens < 1) return 0;
  const int64_t a = 8 * max_model_len, b = 4 * max_num_seqs * (int64_t)page_tokens;
  const int64_t w = a > b ? a : b;
  return w < 64 * 1024 ? w : 64 * 1024;
}

extern "C" int64_t mla_plan_context_chunks(const int32_t* context_lens, int32_t B, int64_t row_budget,
                                           int32_t* chunk_starts, int32_t* chunk_lens, int64_t max_chunks) {
  if (B < 0 || (B > 0 && !context_lens)) return -(int64_t)MLA_ERR_NULL;
  if (row_budget < mla::kPage || row_budget > INT32_MAX) return -(int64_t)MLA_ERR_SHAPE;
  if (max_chunks < 0 || (max_chunks > 0 && (!chunk_starts || !chunk_lens))) return -(int64_t)MLA_ERR_NULL;
  int64_t n_chunks = 0, used = 0;
  bool open = false;                       // the current chunk holds a piece
  auto put = [&](int32_t b, int64_t start, int64_t take) {
    if (!open) {
      if (n_chunks < max_chunks) {
        for (int32_t k = 0; k < B; ++k) {
          chunk_starts[n_chunks * B + k] = 0;
          chunk_lens[n_chunks * B + k] = 0;
        }
      }
      open = true;
    }
    if (n_chunks < max_chunks) {
      chunk_starts[n_chunks * B + b] = (int32_t)start;
      chunk_lens[n_chunks * B + b] = (int32_t)take;
    }
  };
  for (int32_t b = 0; b < B; ++b) {
    const int64_t n = context_lens[b] > 0 ? context_lens[b] : 0;
    int64_t pos = 0;
    while (pos < n) {
      const int64_t room = row_budget - used;
      const int64_t take = n - pos <= room ? n - pos : room / mla::kPage * mla::kPage;
      if (take == 0) {                    // no whole page left: close the chunk
        ++n_chunks;
        open = false;
        used = 0;
        continue;
      }
      put(b, pos, take);
      used += take;
      pos += take;
    }
  }
  if (open) ++n_chunks;
  return n_chunks;
}
