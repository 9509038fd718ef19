// Prefill of new tokens, the compute-friendly MLA path: multi-head attention with
// 192-wide keys [k_nope[s,h] | k_pe[s]] (the one rope key shared by every head) and
// 128-wide values, ragged causal requests, output plus natural-log LSE so that a
// context part can be merged in with mla_merge_attn_states.
// Source: "vLLM 源码完全拆解(三十七):MLA 注意力后端", §两套算法 (compute-friendly form
// for prefill, softmax scale 1/sqrt(192)) and §Prefill (run_prefill_new_tokens: keys
// and values from kv_b_proj, k_pe broadcast over heads, causal over the new tokens
// after the request's context).
//
// One workgroup per (64 query rows, head, request); wave w owns 16 query rows.  Keys
// stream in blocks of 64: the block's keys are staged row-major in LDS (the A operand
// of the score MFMAs: 16 keys x 32 features per lane group), its values transposed
// (the A operand of the PV MFMAs: 16 features x 8 keys).  The query rows stay in
// registers as the B operand, so the scores come out as S^T (keys x queries) and each
// lane holds 16 scores of one query: the row max and sum need two xor shuffles.  The
// softmax is the online one: running max and sum per row, O rescaled when the max
// grows.  The PV contraction pairs the lane's own probabilities with the values in a
// permuted key order (its k index 8g+e is key 4g+e of the first 16-key tile of the
// step for e < 4, key 4g+e-4 of the second for e >= 4), the same on both operands.
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

constexpr int kPQ = 64;              // query rows per workgroup
constexpr int kPK = 64;              // keys per block
constexpr int kKPitch = 192 + 8;     // bf16 per staged key row (400 B: 16 rows on distinct banks)
constexpr int kVtPitch = kPK + 8;    // bf16 per transposed value row (144 B)

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void prefill_mha_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) char smem[(kPK * kKPitch + 128 * kVtPitch) * 2];
  MLA_LDS char* lds = (MLA_LDS char*)(smem);
  MLA_LDS uint16_t* ks = reinterpret_cast<MLA_LDS uint16_t*>(lds);
  MLA_LDS uint16_t* vt = reinterpret_cast<MLA_LDS uint16_t*>(lds + kPK * kKPitch * 2);
  const int b = blockIdx.z, h = blockIdx.y;
  // request bounds, clamped into the buffers whatever the caller passed
  const int64_t q0 = min<int64_t>(max<int64_t>(p.cu_q[b], 0), p.T);
  const int64_t q1 = min<int64_t>(max<int64_t>(p.cu_q[b + 1], q0), p.T);
  const int64_t k0 = min<int64_t>(max<int64_t>(p.cu_k[b], 0), p.S);
  const int64_t k1 = min<int64_t>(max<int64_t>(p.cu_k[b + 1], k0), p.S);
  const int qlen = (int)min<int64_t>(q1 - q0, 0x7fffffff), klen = (int)min<int64_t>(k1 - k0, 0x7fffffff);
  const int qb = blockIdx.x * kPQ;
  if (qb >= qlen) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, l16 = l & 15;

  // this lane's query row: the B-operand column of the score MFMAs
  const int qi = qb + 16 * w + l16;
  const bool q_ok = qi < qlen;
  const uint16_t* qrow = p.q + (q0 + (q_ok ? qi : 0)) * p.q_st + (int64_t)h * p.q_sh;
  bf16x8_t qf[6];
#pragma unroll
  for (int kk = 0; kk < 6; ++kk) qf[kk] = *reinterpret_cast<const bf16x8_t*>(qrow + 32 * kk + 8 * g);

  const int ctx = klen - qlen;
  const int last_row = min(qb + kPQ, qlen) - 1;
  const int kend = p.causal ? max(0, min(klen, ctx + last_row + 1)) : klen;
  const int nvis = p.causal ? max(0, min(klen, ctx + qi + 1)) : klen;

  float m = -INFINITY, lsum = 0.f;
  f32x4_t o[8];
#pragma unroll
  for (int ft = 0; ft < 8; ++ft) o[ft] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // keys kb .. kb+63: 24 chunks of 16 B per key row (16 of k_nope, 8 of k_pe) and
  // 16 chunks per value row; rows past the request read as zeros.  (Loading the next
  // block during the current one's MFMAs measured no faster and cost the registers
  // that three waves per SIMD need.)
  u32x4_t kv[6], vv[2][2];
  auto load_block = [&](int kb) {
#pragma unroll
    for (int j = 0; j < 6; ++j) {
      const int i = tid + 256 * j;
      const int r = i / 24, c = i % 24;
      const int key = kb + r;
      const uint16_t* src = c < 16 ? p.kn + (k0 + key) * p.kn_st + (int64_t)h * p.kn_sh + c * 8
                                   : p.kp + (k0 + key) * p.kp_st + (c - 16) * 8;
      kv[j] = key < klen ? *reinterpret_cast<const u32x4_t*>(src) : u32x4_t{0u, 0u, 0u, 0u};
    }
    // values: a lane takes one 16-byte chunk (8 features) of two adjacent keys, so
    // that the transposed rows get 4-byte writes (the two keys' values of one
    // feature); lanes 0..31 of a wave cover the 32 key pairs of one chunk, lanes
    // 32..63 the next chunk: 64 distinct banks per write instruction
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int kp = l & 31, c = 2 * (2 * w + j) + (l >> 5);
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const int key = kb + 2 * kp + d;
        vv[j][d] = key < klen
                       ? *reinterpret_cast<const u32x4_t*>(p.v + (k0 + key) * p.v_st + (int64_t)h * p.v_sh + c * 8)
                       : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  };
  for (int kb = 0; kb < kend; kb += kPK) {
    load_block(kb);
    lds_barrier();                                      // the previous block's reads are done
#pragma unroll
    for (int j = 0; j < 6; ++j) {
      const int i = tid + 256 * j;
      *reinterpret_cast<MLA_LDS u32x4_t*>(lds + (i / 24) * kKPitch * 2 + (i % 24) * 16) = kv[j];
    }
    MLA_LDS uint32_t* vt32 = reinterpret_cast<MLA_LDS uint32_t*>(vt);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int kp = l & 31, c = 2 * (2 * w + j) + (l >> 5);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // features c*8 + 2e and c*8 + 2e + 1 of keys 2kp, 2kp + 1
        const uint32_t a = vv[j][0][e], b = vv[j][1][e];
        vt32[((c * 8 + 2 * e) * kVtPitch) / 2 + kp] = (a & 0xFFFFu) | (b << 16);
        vt32[((c * 8 + 2 * e + 1) * kVtPitch) / 2 + kp] = (a >> 16) | (b & 0xFFFF0000u);
      }
    }
    lds_barrier();

    // S^T: four 16-key tiles; s[kt][r] = score of key kb + 16kt + 4g + r, query l16
    f32x4_t s[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      s[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 6; ++kk) {
        const bf16x8_t a = *reinterpret_cast<const MLA_LDS bf16x8_t*>(ks + (16 * kt + l16) * kKPitch + 32 * kk + 8 * g);
        s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[kk], s[kt], 0, 0, 0);
      }
    }
    float bmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kb + 16 * kt + 4 * g + r;
        const float x = key < nvis ? s[kt][r] * p.scale_log2 : -INFINITY;
        s[kt][r] = x;
        bmax = fmaxf(bmax, x);
      }
    }
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16, 64));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
    const float mn = fmaxf(m, bmax);
    const float alpha = mn == -INFINITY ? 1.f : exp2f(m - mn);
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pr = mn == -INFINITY ? 0.f : exp2f(s[kt][r] - mn);
        s[kt][r] = pr;
        psum += pr;
      }
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    lsum = lsum * alpha + psum;
    m = mn;
#pragma unroll
    for (int ft = 0; ft < 8; ++ft) o[ft] *= alpha;

    // O^T += V^T P^T: k step c pairs tiles 2c and 2c + 1
    bf16x8_t pb[2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
      pb[c] = bf16x8_t{(__bf16)s[2 * c][0], (__bf16)s[2 * c][1], (__bf16)s[2 * c][2], (__bf16)s[2 * c][3],
                       (__bf16)s[2 * c + 1][0], (__bf16)s[2 * c + 1][1], (__bf16)s[2 * c + 1][2],
                       (__bf16)s[2 * c + 1][3]};
#pragma unroll
    for (int ft = 0; ft < 8; ++ft) {
      const MLA_LDS uint16_t* vrow = vt + (16 * ft + l16) * kVtPitch;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16x4_t lo = *reinterpret_cast<const MLA_LDS bf16x4_t*>(vrow + 32 * c + 4 * g);
        const bf16x4_t hi = *reinterpret_cast<const MLA_LDS bf16x4_t*>(vrow + 32 * c + 16 + 4 * g);
        const bf16x8_t a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[ft] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[c], o[ft], 0, 0, 0);
      }
    }
  }

  // o[ft][r] = O[query l16][feature 16ft + 4g + r]
  if (q_ok) {
    const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
    uint16_t* orow = p.out + (q0 + qi) * p.o_st + (int64_t)h * p.o_sh;
#pragma unroll
    for (int ft = 0; ft < 8; ++ft) {
      const bf16x4_t v4 = {(__bf16)(o[ft][0] * inv), (__bf16)(o[ft][1] * inv), (__bf16)(o[ft][2] * inv),
                           (__bf16)(o[ft][3] * inv)};
      *reinterpret_cast<bf16x4_t*>(orow + 16 * ft + 4 * g) = v4;
    }
    if (g == 0)
      p.lse[(q0 + qi) * p.N + h] = lsum > 0.f ? (m + __log2f(lsum)) * 0.6931471805599453f : -INFINITY;
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
  const dim3 grid((unsigned)((max_q_len + kPQ - 1) / kPQ), (unsigned)N, (unsigned)B);
  hipLaunchKernelGGL(prefill_mha_kernel, grid, dim3(256), 0, reinterpret_cast<hipStream_t>(stream), p);
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
