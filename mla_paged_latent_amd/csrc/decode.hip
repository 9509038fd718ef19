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
//   split plan           computed inside the decode kernels from seq_lens: the batch is
//                        cut into equal-cost streams of (request, token range) pieces,
//                        one per workgroup and head group
//   decode_wide_kernel   q_len * N > 16: one work unit = (stream, head group of 64
//                        query rows); each piece's cache rows stream through
//                        LDS in 32-token blocks (global->LDS DMA ring) and every query
//                        row of the group scores against each staged block:
//                          S^T = K . Q^T   (MFMA; 4 score waves, each 32 rows x 16
//                                           tokens, Q in registers)
//                          softmax in the log2 domain against a fixed reference max
//                          O^T += V^T . P^T (MFMA; 4 value waves, each 128 latent features
//                                            of all rows, V^T via LDS transpose reads, P
//                                            via LDS), one block behind the scores
//   decode_narrow_kernel q_len * N <= 16 (16-head decode): 16 rows per unit, whole
//                        pages double-buffered, the 4 waves split each page's tokens
//   Both write the final output (single split) or float32 partials; then
//   merge_kernel         LSE-weighted combine of the partials of split requests
#include <atomic>
#include <type_traits>
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
  int32_t m_wg;        // query rows per work unit (16 narrow, 64 wide)
  int32_t hg_heads;    // heads per head group = m_wg / q_len
  float scale_log2;    // softmax_scale * log2(e)
  uint16_t* out;
  int64_t o_sb, o_st, o_sh;
  float* lse;
  // workspace views
  int4* req;           // per request: {first partial slot, pieces, 0, clamped seq_len}
  float* part_lse;     // [slots * n_hg * m_wg]
  float* part_o;       // [slots * n_hg * m_wg * 512]
  int32_t num_splits;  // 0 automatic, k >= 1 forced
  int32_t n_streams;   // streams of the plan
  int32_t n_units;     // n_streams x head groups, rounded for the sibling order
  int32_t max_slots;   // partial slots the workspace holds
};

// unit -> (stream, head group).  Sibling head groups of one stream sit 8 units apart
// so that, with a grid that is a multiple of 8, they run at the same time on the same
// XCD (workgroups are dispatched round-robin over the 8 XCDs) and share the stream's
// pages through that XCD's L2.
__device__ __forceinline__ void unit_to_stream(int u, int n_hg, int* stream, int* hg) {
  if (n_hg == 1) {
    *stream = u;
    *hg = 0;
  } else {
    *stream = (u / (8 * n_hg)) * 8 + (u & 7);
    *hg = (u >> 3) % n_hg;
  }
}

// ---------------------------------------------------------------------------
// Split plan ([vLLM-MLA] §FlashMLA: the split count follows seq_len and the number
// of compute units; single-partition mode for batch invariance)
// ---------------------------------------------------------------------------
// A stream is the ordered list of (request, token range) pieces one unit works
// through; a unit is (stream, head group).
//
// num_splits == 0 (automatic): request b occupies a stretch of kSegOverhead +
// pages(b) cost positions on one line (the overhead stands for the fixed cost of
// a piece: its start-up and its partial row); the line is cut into n_streams
// streams, stream s covering [s * total / n, (s + 1) * total / n), one unit per
// workgroup and head group, so that every workgroup gets the same amount of work
// (within one position) whatever the length mix.  The pages of b that fall in stream
// s form one piece; b is split when its stretch straddles a cut.  The piece of b in
// stream s writes partial slot b + s: the slots of b + 1 all lie above those of b,
// so B + n_streams slots suffice.  Every workgroup derives the plan from seq_lens
// itself (one prefix sum over the batch), so there is no planning launch and no
// host synchronisation.
//
// num_splits == k >= 1: stream s is split s % k of request s / k, over page-aligned
// chunks of ceil(seq / k) tokens; its partial slot is s.  k == 1 keeps one piece
// per request (bit-identical results whatever the rest of the batch).
//
// The piece that holds a request's first page (head group 0) records
// {first slot, number of pieces} in req[b] for the merge.
constexpr int kSegOverhead = 4;                         // in pages
constexpr int32_t kMaxPagesPerSeq = 0x7fffffff / kPage;  // block-table entries a request can reach

__device__ __forceinline__ int clamp_seq(int s, int cap) { return s < 0 ? 0 : (s > cap ? cap : s); }
__device__ __forceinline__ int pages_of(int s) { return (s + kPage - 1) / kPage; }

// LDS scratch of the planner: 256 exclusive prefixes, 4 wave totals, a 3-value result
constexpr int kPlanLdsBytes = (256 + 4 + 4) * 8;

// a workgroup-uniform 64-bit value read from LDS, moved to scalar registers
__device__ __forceinline__ long long uniform64(long long v) {
  const uint64_t u = (uint64_t)v;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (long long)(((uint64_t)hi << 32) | lo);
}

// 64-bit division for the rare plans whose products overflow 32 bits, as a compact
// bit-serial loop: the plan divides at several places, and the usual inlined 64-bit
// sequence at each of them would bloat the kernels' code.  Only the kernels built for
// such batches (P64) contain it; the host picks them when a bound on the plan's
// products (batch size, block-table width and stream count) exceeds 32 bits.
__device__ __forceinline__ uint64_t udiv64_slow(uint64_t a, uint64_t b) {
  uint64_t q = 0, r = 0;
#pragma unroll 1
  for (int i = 63; i >= 0; --i) {
    r = (r << 1) | ((a >> i) & 1u);
    if (r >= b) {
      r -= b;
      q |= 1ull << i;
    }
  }
  return q;
}

template <bool P64>
struct PlanTotals {
  long long total;    // cost positions of the whole batch (>= 1)
  long long n;        // streams
  // 64-bit division is a long software sequence on the GPU: when every product below
  // fits in 32 bits (any realistic batch), 32-bit unsigned division is used instead
  __device__ __forceinline__ bool small() const {
    return !P64 || total <= (long long)(0xFFFFFFFFu / (uint32_t)(n + 1));
  }
  __device__ __forceinline__ long long start(long long s) const {
    if (small()) return (long long)((uint32_t)s * (uint32_t)total / (uint32_t)n);
    return (long long)udiv64_slow((uint64_t)(s * total), (uint64_t)n);
  }
  // the stream holding position X: the largest s with start(s) <= X
  __device__ __forceinline__ int stream_of(long long X) const {
    if (small()) return (int)((((uint32_t)X + 1u) * (uint32_t)n - 1u) / (uint32_t)total);
    return (int)udiv64_slow((uint64_t)((X + 1) * n - 1), (uint64_t)total);
  }
};

// Thread tid < 256 sums the costs of requests [tid * K, tid * K + K), K = ceil(B / 256);
// pre[tid] receives the exclusive prefix of those sums (threads 256 and up of a larger
// workgroup own no requests and only take part in the barriers).
// *seq0 receives the clamped seq_len of request tid * K (0 if there is none).
template <bool P64>
__device__ __forceinline__ PlanTotals<P64> plan_prefix(const DecodeParams& p, MLA_LDS long long* pre, int tid, int* seq0) {
  const int cap = p.max_pages * kPage;
  const int K = (p.B + 255) >> 8;
  const int b0 = tid * K;
  const int b1 = b0 + K < p.B ? b0 + K : p.B;
  long long local = 0;
  *seq0 = 0;
  for (int b = b0; b < b1; ++b) {
    const int s = clamp_seq(p.seq_lens[b], cap);
    if (b == b0) *seq0 = s;
    local += kSegOverhead + pages_of(s);
  }
  const int l = tid & 63;
  long long incl = local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const long long v = __shfl_up(incl, d, 64);
    if (l >= d) incl += v;
  }
  MLA_LDS long long* wtot = pre + 256;
  if (l == 63 && tid < 256) wtot[tid >> 6] = incl;
  lds_barrier();
  long long off = 0;
  for (int k = 0; k < (tid >> 6); ++k) off += wtot[k];
  if (tid < 256) pre[tid] = off + incl - local;
  PlanTotals<P64> r;
  r.total = uniform64(wtot[0] + wtot[1] + wtot[2] + wtot[3]);
  // no more streams than positions, so that no stream is empty (the pieces of a
  // request then sit in consecutive streams)
  r.n = p.n_streams < r.total ? p.n_streams : r.total;
  lds_barrier();
  return r;
}

// The request holding cost position X (< total), the position where it starts and its
// clamped seq_len (seq0: this thread's value from plan_prefix).
__device__ __forceinline__ void plan_find(const DecodeParams& p, MLA_LDS long long* pre, long long X, long long total,
                                          int tid, int seq0, int* b_out, long long* c_out, int* seq_out) {
  MLA_LDS long long* sel = pre + 260;
  const int cap = p.max_pages * kPage;
  const int K = (p.B + 255) >> 8;
  const int b0 = tid * K;
  const int b1 = b0 + K < p.B ? b0 + K : p.B;
  const long long e0 = tid < 256 ? pre[tid] : total;
  const long long e1 = tid < 255 ? pre[tid + 1] : total;
  if (b0 < b1 && e0 <= X && X < e1) {
    long long c = e0;
    int b = b0, sq = seq0;
    for (; b < b1 - 1; ++b) {
      const long long cb = kSegOverhead + pages_of(sq);
      if (X < c + cb) break;
      c += cb;
      sq = clamp_seq(p.seq_lens[b + 1], cap);
    }
    sel[0] = b;
    sel[1] = c;
    sel[2] = sq;
  }
  lds_barrier();
  *b_out = __builtin_amdgcn_readfirstlane((int)sel[0]);
  *c_out = uniform64(sel[1]);
  *seq_out = __builtin_amdgcn_readfirstlane((int)sel[2]);
  lds_barrier();                                        // sel is rewritten by the next search
}

// floor(x * np / len) for 0 <= x <= len (32-bit arithmetic when the product fits)
template <bool P64>
__device__ __forceinline__ int scale_floor(int x, int np, int len) {
  if (!P64 || (uint64_t)(uint32_t)len * (uint32_t)np <= 0xFFFFFFFFull)
    return (int)((uint32_t)x * (uint32_t)np / (uint32_t)len);
  return (int)udiv64_slow((uint64_t)x * (uint64_t)np, (uint64_t)len);
}

// One piece of a stream: request b, tokens [t_begin, t_end) of its seq (clamped)
// tokens, the number of pieces of b and this piece's partial slot.
struct Piece {
  int b, t_begin, t_end, seq, nsplit, slot;
};

// Walks the pieces of stream s in order; every value is workgroup-uniform.  pre / tot
// come from plan_prefix (automatic mode only).
template <bool P64>
struct PieceIter {
  long long lo, hi, c;
  PlanTotals<P64> tot;
  int b, s;
  int seq_b;          // clamped seq_len of request b as found by plan_find (-1: unknown)
  bool done;

  __device__ __forceinline__ void init(const DecodeParams& p, MLA_LDS long long* pre, const PlanTotals<P64>& tot, int stream,
                                       int tid, int seq0) {
    s = stream;
    done = false;
    seq_b = -1;
    if (p.num_splits > 0) return;
    this->tot = tot;
    lo = tot.start(s);
    hi = tot.start(s + 1);
    if (s >= tot.n) {
      done = true;
      return;
    }
    plan_find(p, pre, lo, tot.total, tid, seq0, &b, &c, &seq_b);
  }

  __device__ __forceinline__ bool next(const DecodeParams& p, int hg, int tid, Piece& pc) {
    if (done) return false;
    const int cap = p.max_pages * kPage;
    if (p.num_splits > 0) {
      done = true;
      const int k = p.num_splits;
      const int rb = s / k, sp = s - rb * k;
      const int seq = clamp_seq(p.seq_lens[rb], cap);
      int chunk = pages_of((seq + k - 1) / k) * kPage;
      if (chunk < kPage) chunk = kPage;
      const int ns = seq > 0 ? (seq + chunk - 1) / chunk : 1;
      if (sp == 0 && hg == 0 && tid == 0) p.req[rb] = make_int4(rb * k, ns, 0, seq);
      if (sp >= ns) return false;
      const int t0 = sp * chunk;
      const int t1 = t0 + chunk < seq ? t0 + chunk : seq;
      pc = Piece{rb, t0, t1 > t0 ? t1 : t0, seq, ns, s};
      return true;
    }
    while (b < p.B && c < hi) {
      const int seq = seq_b >= 0 ? seq_b : clamp_seq(p.seq_lens[b], cap);
      seq_b = -1;
      const int np = pages_of(seq);
      const int len = kSegOverhead + np;                // b's stretch: [c, c + len)
      bool have = false;
      if (np == 0) {
        if (c >= lo) {
          if (hg == 0 && tid == 0) p.req[b] = make_int4(0, 1, 0, 0);
          pc = Piece{b, 0, 0, 0, 1, b + s};
          have = true;
        }
      } else {
        // Where the stretch maps onto the pages.  Usually b starts inside a stream that
        // also holds the end of an earlier request: that stream pays b's extra piece, so
        // the overhead stands at the front and relative position x ends page x - O.  When
        // a cut falls exactly on b's start, no stream pays an extra piece for b, and the
        // stretch maps in proportion instead (x ends page floor(x * np / len)), so that a
        // request cut into k streams gives each the same share of its pages.  Page 0 lies
        // in stream sf, page np - 1 in stream sl.  A stream strictly between them with no
        // page of b (only possible in proportion, for streams shorter than len / np
        // positions) still takes an empty piece, a partial of weight zero, so that b has
        // a partial in every slot it uses.
        const bool prop = tot.start(tot.stream_of(c)) == c;
        const int first_end = prop ? (len + np - 1) / np : kSegOverhead + 1;
        const int sf = tot.stream_of(c + first_end - 1), sl = tot.stream_of(c + len - 1);
        if (s >= sf && s <= sl) {
          const int xa = lo > c ? (int)(lo - c) : 0;
          const int xe = hi < c + len ? (int)(hi - c) : len;
          const int pa = prop ? scale_floor<P64>(xa, np, len) : (xa > kSegOverhead ? xa - kSegOverhead : 0);
          const int pe = prop ? scale_floor<P64>(xe, np, len) : (xe > kSegOverhead ? xe - kSegOverhead : 0);
          if (s == sf && hg == 0 && tid == 0) p.req[b] = make_int4(b + sf, sl - sf + 1, 0, seq);
          const int t0 = pa * kPage < seq ? pa * kPage : seq;
          const int t1 = pe * kPage < seq ? pe * kPage : seq;
          pc = Piece{b, t0, t1, seq, sl - sf + 1, b + s};
          have = true;
        }
      }
      c += len;
      ++b;
      if (have) return true;
    }
    done = true;
    return false;
  }
};

// ---------------------------------------------------------------------------
// Block staging
// ---------------------------------------------------------------------------
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

// The cache rows of a piece stream through LDS in 32-token blocks (half a page).  A
// block is stored column-group major: group G = c >> 3 (128 bytes of every row, 4 KB)
// holds 32 tokens x 8 chunks of 16 B, chunk c of token t at slot
// G * 256 + t * 8 + ((c & 7) ^ s(t)).  bf16 blocks land straight in a 4-slot ring;
// fp8 blocks land raw in a 4-slot ring and are converted into 2 bf16 slots plus
// per-token factors.  Ring slot of a block = its index in the unit's block stream & 3.
constexpr int kBlk = 32;
constexpr int kBlkBytesBf16 = kBlk * kRowBytesBf16;    // 36864
constexpr int kBlkBytesFp8 = kBlk * kRowBytesFp8;      // 18688
constexpr int kBlkGroupBytes = kBlk * 128;             // 4096: one 128-byte column of the block
constexpr int kBlkChunksFp8 = kBlkBytesFp8 / 16;       // 1168
constexpr int kRing = 4;                               // DMA ring depth (blocks)
constexpr int kSlot = kBlkBytesBf16;                   // bf16 block slots at 0, 36864, ...
constexpr int kRaw = 2 * kSlot;                        // fp8: 2 converted slots, then 4 raw blocks
constexpr int kFac = kRaw + kRing * kBlkBytesFp8;      // fp8 per-token factors, 2 x [3][32] f32
constexpr int kFacBytes = 3 * kBlk * 4;
constexpr int kStageEnd = 149504;                      // end of the staging area
static_assert(kRing * kSlot <= kStageEnd && kFac + 2 * kFacBytes <= kStageEnd, "staging LDS plan");

// bf16 block: 36 DMA instructions of 64 x 16 B; wave w loads tokens 8w .. 8w+7 of
// every 128-byte column i (instruction i = 0..8): lane j takes token t = 8w + (j >> 3),
// chunk 8i + ((j & 7) ^ s(t)), so the global offset is voff + 128 i and the LDS
// destination 1024 w + 4096 i.
template <int... I>
__device__ __forceinline__ void issue_blk_bf16_seq(std::integer_sequence<int, I...>, const char* blk,
                                                   uint32_t voff, uint32_t lds) {
  (dma_16B<128 * I, kBlkGroupBytes * I>(blk, voff, lds), ...);
}

__device__ __forceinline__ void issue_blk_bf16(const char* blk, MLA_LDS char* dst, int w, int l) {
  const int t = 8 * w + (l >> 3);
  const uint32_t voff = (uint32_t)(t * kRowBytesBf16 + ((l & 7) ^ page_swz(t)) * 16);
  issue_blk_bf16_seq(std::make_integer_sequence<int, 9>{}, blk, voff, lds_addr(dst) + 1024u * (uint32_t)w);
}

// fp8 block: the 18688 raw bytes as 1168 flat 16-byte chunks, instructions
// k = w + 4i (i = 0..4) while k * 64 + lane < 1168.
template <int I>
__device__ __forceinline__ void issue_blk_fp8_one(const char* blk, uint32_t voff, uint32_t lds, int w, int l) {
  if ((w + 4 * I) * 64 + l < kBlkChunksFp8) dma_16B<0, 4096 * I>(blk + 4096 * I, voff, lds);
}

template <int... I>
__device__ __forceinline__ void issue_blk_fp8_seq(std::integer_sequence<int, I...>, const char* blk,
                                                  uint32_t voff, uint32_t lds, int w, int l) {
  (issue_blk_fp8_one<I>(blk, voff, lds, w, l), ...);
}

__device__ __forceinline__ void issue_blk_fp8(const char* blk, MLA_LDS char* dst, int w, int l) {
  issue_blk_fp8_seq(std::make_integer_sequence<int, 5>{}, blk, (uint32_t)(1024 * w + 16 * l),
                    lds_addr(dst) + 1024u * (uint32_t)w, w, l);
}

// Rows >= valid of this wave's own DMA share (tokens 8w .. 8w+7 of every column)
// become zero: cache bytes past the end of a sequence may hold anything, and a
// NaN there times a zero weight would still reach O.
__device__ __forceinline__ void zero_own_tail(MLA_LDS char* blk, int valid, int w, int l) {
  if (8 * w + 8 > valid && 8 * w + (l >> 3) >= valid) {
#pragma unroll
    for (int i = 0; i < 9; ++i)
      *reinterpret_cast<MLA_LDS u32x4_t*>(blk + kBlkGroupBytes * i + 1024 * w + 16 * l) = u32x4_t{0u, 0u, 0u, 0u};
  }
}

// fp8 raw block -> swizzled bf16 block (exact) plus the per-token factors
// {k_scale * softmax scale * log2 e, v_scale, 1 / v_scale}; rows >= valid become 0.
__device__ __forceinline__ void convert_fp8_blk(const MLA_LDS char* raw, MLA_LDS char* conv,
                                                MLA_LDS float* fac, int valid, int tid, float scale_log2) {
  // thread tid converts chunk 8i + ((tid & 7) ^ s(t)) of token t = tid >> 3 for i = 0..8
  // (output slot tid + 256 i); the nine 8-byte code reads are issued together so their
  // LDS latency is paid once
  const int t = tid >> 3;
  const bool ok = t < valid;
  const MLA_LDS char* src = raw + t * kRowBytesFp8 + ((tid & 7) ^ page_swz(t)) * 8;
  u32x2_t code[kChunksPerRow / 8];
#pragma unroll
  for (int i = 0; i < kChunksPerRow / 8; ++i)
    code[i] = ok ? *reinterpret_cast<const MLA_LDS u32x2_t*>(src + 64 * i) : u32x2_t{0u, 0u};
#pragma unroll
  for (int i = 0; i < kChunksPerRow / 8; ++i) {
    const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)code[i][0], 1.0f, false);
    const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)code[i][0], 1.0f, true);
    const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)code[i][1], 1.0f, false);
    const bf16x2_t e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)code[i][1], 1.0f, true);
    *reinterpret_cast<MLA_LDS bf16x8_t*>(conv + (tid + 256 * i) * 16) =
        bf16x8_t{a[0], a[1], b[0], b[1], d[0], d[1], e[0], e[1]};
  }
  if (tid < kBlk) {
    float k = 0.f, v = 0.f;
    if (tid < valid) {
      const f32x2_t sc = *reinterpret_cast<const MLA_LDS f32x2_t*>(raw + tid * kRowBytesFp8 + kRow);
      k = sc[0];
      v = sc[1];
    }
    fac[tid] = k * scale_log2;
    fac[kBlk + tid] = v;
    fac[2 * kBlk + tid] = v != 0.f ? 1.0f / v : 0.f;
  }
}

// ---------------------------------------------------------------------------
// Softmax reference max
// ---------------------------------------------------------------------------
// Softmax bookkeeping without rescaling the accumulators.  Each row's reference
// max m is fixed from the first 32-token block of the unit (exact for that block);
// later scores may exceed it, so p = 2^(s - m) can be > 1, which float32
// accumulation and bfloat16 probabilities represent without loss of relative
// precision.  A visible score more than kRefSlack above m would risk overflow:
// the block then raises a flag and the workgroup redoes the unit with the larger
// reference.  O never needs a VALU rescale inside the page loop.
constexpr float kRefSlack = 64.0f;

// ---------------------------------------------------------------------------
// Narrow variant: 16 query rows per unit (16-head decode), 4 waves, 32-token blocks
// ---------------------------------------------------------------------------
// Division of labour inside a workgroup (w = wave, th = w & 1):
//  * scores: wave w computes S^T = K . Q^T for tokens 16th .. 16th+15 of each block and
//    all 16 rows (16x16x32 MFMA, K fragments from LDS, the query in registers).  Waves
//    w and w ^ 2 compute the same scores: that costs LDS and MFMA time the block's HBM
//    time covers, and keeps one barrier per block.  Waves 0 and 1 write the weights P.
//  * values: wave w owns latent features 128w .. 128w+127 of the 16 rows,
//    O^T += V^T . P^T on 16x16x32 MFMA over the block's 32 tokens.
// The contraction order of the 32 tokens inside one PV MFMA is a permutation chosen so
// that each transpose read touches 8 consecutive tokens per half-wave (conflict-free
// with the block swizzle); P is stored in that order, so the product is unchanged.
// The unit's pieces form one block stream: the DMA of the next piece's first blocks is
// issued while the current piece finishes, so a piece boundary costs no page latency.
constexpr int kNRows = 16;
constexpr int kNP = kStageEnd;                         // P: 2 buffers x 16 rows x 64 B
constexpr int kNPBytes = kNRows * 64;
constexpr int kNStats = kNP + 2 * kNPBytes;            // per token half and row {m, l, lr, -}
constexpr int kNFlag = kNStats + 2 * kNRows * 16;      // overflow flag of the reference max
constexpr int kNPlan = kNFlag + 16;                    // split-plan scratch
constexpr int kNLdsBytes = kNPlan + kPlanLdsBytes;
static_assert(kNLdsBytes <= 160 * 1024, "LDS budget");

// LDS row of query row R in a P buffer: bits 0, 1 XORed with bits 2, 3, so that rows
// differing only in bits 2, 3 fall in different quarters of the banks
__device__ __forceinline__ int p_row(int R) { return R ^ ((R >> 2) & 3); }


// token of k-slot 4h + i (i = 0..3) of lane group g in the PV contraction
__device__ __forceinline__ int pv_token(int g, int h) { return 16 * (g >> 1) + 8 * h + 4 * (g & 1); }

// S^T of this wave's 16 tokens for the 16 rows: 18 steps of 32 features, K fragments
// read kPrefK steps ahead.
__device__ __forceinline__ f32x4_t narrow_scores(const MLA_LDS char* blk, const bf16x8_t (&qf)[18],
                                                 const uint32_t (&kbase)[2]) {
  constexpr int kPrefK = 4;
  uint32_t ka[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) ka[m] = opaque(lds_addr(blk) + kbase[m]);
  bf16x8_t kbuf[kPrefK];
#pragma unroll
  for (int d = 0; d < kPrefK; ++d) kbuf[d] = lds_read_b128_at(ka[d & 1] + (d >> 1) * kBlkGroupBytes);
  f32x4_t sc = {};
#pragma unroll
  for (int kk = 0; kk < 18; ++kk) {
    const bf16x8_t a = kbuf[kk % kPrefK];
    const int nk = kk + kPrefK;
    if (nk < 18) kbuf[kk % kPrefK] = lds_read_b128_at(ka[nk & 1] + (nk >> 1) * kBlkGroupBytes);
    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[kk], sc, 0, 0, 0);
  }
  return sc;
}

// O^T[this wave's 128 features][16 rows] += V^T . P^T over one block: 8 feature tiles of
// 16, each one MFMA over the 32 tokens (two transpose reads for V^T); P^T is one 16-byte
// read per lane.
__device__ __forceinline__ void narrow_pv(const MLA_LDS char* blk, const MLA_LDS char* pbuf, f32x4_t (&o)[8],
                                          const uint32_t (&vbase)[2][4], uint32_t pbase) {
  uint32_t va[2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int f3 = 0; f3 < 4; ++f3) va[h][f3] = opaque(lds_addr(blk) + vbase[h][f3]);
  const bf16x8_t pb = lds_read_b128_at(opaque(lds_addr(pbuf) + pbase));
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    const uint32_t off = (uint32_t)((f >> 2) * kBlkGroupBytes);
    const bf16x4_t lo = lds_read_tr16_at(va[0][f & 3] + off);
    const bf16x4_t hi = lds_read_tr16_at(va[1][f & 3] + off);
    const bf16x8_t a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    o[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, o[f], 0, 0, 0);
  }
}

// A piece whose blocks are (being) staged: token range, page range and page ids.
struct StagedPiece {
  Piece pc;
  int nblk, pg0, pg1;
  PageIds ids;
};

// (the piece values are workgroup-uniform; readfirstlane states it to the compiler)
__device__ __forceinline__ void stage_piece(StagedPiece& sp, const DecodeParams& p, int l) {
  sp.pc.b = __builtin_amdgcn_readfirstlane(sp.pc.b);
  sp.pc.t_begin = __builtin_amdgcn_readfirstlane(sp.pc.t_begin);
  sp.pc.t_end = __builtin_amdgcn_readfirstlane(sp.pc.t_end);
  sp.nblk = sp.pc.t_end > sp.pc.t_begin ? (sp.pc.t_end - sp.pc.t_begin + kBlk - 1) / kBlk : 0;
  sp.pg0 = sp.pc.t_begin / kPage;
  sp.pg1 = sp.nblk > 0 ? (sp.pc.t_end + kPage - 1) / kPage : sp.pg0;
  load_page_ids(sp.ids, p, sp.pc.b, sp.pg0, sp.pg1, l);
}

template <bool FP8>
__device__ __forceinline__ void issue_piece_block(StagedPiece& sp, const DecodeParams& p, int jb, int g,
                                                  MLA_LDS char* smem, int w, int l) {
  jb = __builtin_amdgcn_readfirstlane(jb);
  g = __builtin_amdgcn_readfirstlane(g);
  const char* pg = page_ptr(sp.ids, p, sp.pc.b, sp.pg0 + (jb >> 1), sp.pg1, l, FP8);
  if constexpr (FP8)
    issue_blk_fp8(pg + (jb & 1) * kBlkBytesFp8, smem + kRaw + (g & (kRing - 1)) * kBlkBytesFp8, w, l);
  else
    issue_blk_bf16(pg + (jb & 1) * kBlkBytesBf16, smem + (g & (kRing - 1)) * kSlot, w, l);
}

// wait until at most one block (later > 0) or nothing issued after the awaited one is
// outstanding (per-wave instruction counts of a block: 9 bf16; 5, 5, 5, 4 fp8)
template <bool FP8>
__device__ __forceinline__ void wait_blocks_after(int later, int w) {
  if (later <= 0) {
    wait_vmcnt<0>();
  } else if constexpr (FP8) {
    if (w == 3) wait_vmcnt<4>();
    else wait_vmcnt<5>();
  } else {
    wait_vmcnt<9>();
  }
}

// wait until this wave's query and the blocks issued before it have landed, with
// `later` (0, 1 or 2) whole blocks issued after the query still allowed in flight
template <bool FP8>
__device__ __forceinline__ void wait_query_and_block0(int later, int w) {
  if (later <= 0) {
    wait_vmcnt<0>();
  } else if (later == 1) {
    wait_blocks_after<FP8>(1, w);
  } else if constexpr (FP8) {
    if (w == 3) wait_vmcnt<8>();
    else wait_vmcnt<10>();
  } else {
    wait_vmcnt<18>();
  }
}

template <bool FP8, bool P64>
__global__ __launch_bounds__(256, 1) void decode_narrow_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[kNLdsBytes];
  MLA_LDS char* smem = (MLA_LDS char*)(smem_raw);
  const int tid = threadIdx.x;
  const int w = wave_id();
  const int l = lane_id();
  const int th = w & 1;                          // token half of the score phase
  const int l16 = l & 15, g4 = l >> 4;
  MLA_LDS int* ovf_flag = reinterpret_cast<MLA_LDS int*>(smem + kNFlag);
  MLA_LDS f32x4_t* stats = reinterpret_cast<MLA_LDS f32x4_t*>(smem + kNStats);   // [2][16]

  // Per-lane LDS offsets, fixed for the whole kernel.
  // K fragment of step kk: token 16th + l16, chunk 4kk + g4 (group kk >> 1, in-group
  // chunk 4(kk & 1) + g4).
  uint32_t kbase[2];
  {
    const int t = 16 * th + l16;
#pragma unroll
    for (int m = 0; m < 2; ++m) kbase[m] = (uint32_t)(t * 8 + ((4 * m + g4) ^ page_swz(t))) * 16;
  }
  // V^T transpose read h of feature tile f (features 128w + 16f .. +15): the 16 lanes of
  // group g4 read tokens pv_token(g4, h) + (l16 >> 2), features 128w + 16f + 4(l16 & 3)
  // .. +3, i.e. chunk 16w + 2f + ((l16 & 3) >> 1) (group 2w + (f >> 2), in-group chunk
  // 2(f & 3) + ((l16 & 3) >> 1)), byte 8(l16 & 1); f >> 2 only adds an offset.
  uint32_t vbase[2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int f3 = 0; f3 < 4; ++f3) {
      const int t = pv_token(g4, h) + (l16 >> 2);
      const int cin = 2 * f3 + ((l16 & 3) >> 1);
      vbase[h][f3] = (uint32_t)(2 * w * kBlkGroupBytes + (t * 8 + (cin ^ page_swz(t))) * 16 + 8 * (l16 & 1));
    }
  // P rows: 64 B = 4 chunks; chunk g holds the 8 k-slots of lane group g, at position
  // g ^ ((row >> 2) & 3), and row R sits at p_row(R) so that the 8-lane groups of a
  // 16-byte read (rows with equal bits 0, 1) spread over the four quarters of the banks.
  // PV reads chunk g4 of row l16.
  const uint32_t pbase = (uint32_t)(p_row(l16) * 64 + ((g4 ^ ((l16 >> 2) & 3)) * 16));
  // score-phase element i of this lane is token 16th + 4g4 + i = k-slot 4(g4 >> 1) + i of
  // lane group 2th + (g4 & 1)
  const int pg_w = 2 * th + (g4 & 1);
  const uint32_t pwrite = (uint32_t)(p_row(l16) * 64 + ((pg_w ^ ((l16 >> 2) & 3)) * 16) + 8 * (g4 >> 1));

  // query row of this lane in both phases: r = l16
  const int hl = l16 / p.q_len, tq = l16 - hl * p.q_len;
  const int head = hl;                            // one head group
  const bool row_ok = head < p.N;

  MLA_LDS long long* plan_lds = reinterpret_cast<MLA_LDS long long*>(smem + kNPlan);
  PlanTotals<P64> tot{1, 1};
  int seq0 = 0;
  if (p.num_splits == 0) tot = plan_prefix<P64>(p, plan_lds, tid, &seq0);
  for (int u = blockIdx.x; u < p.n_units; u += gridDim.x) {
    int sid, hg;
    unit_to_stream(u, p.n_hg, &sid, &hg);
    if (sid >= p.n_streams) continue;
    PieceIter<P64> it;
    it.init(p, plan_lds, tot, sid, tid, seq0);
    StagedPiece cur, nxt;
    if (!it.next(p, hg, tid, cur.pc)) continue;
    stage_piece(cur, p, l);
    // the following piece is looked up once the current one's first blocks are in flight
    bool nxt_known = false, has_nxt = false;
    auto fetch_nxt = [&]() {
      if (nxt_known) return;
      nxt_known = true;
      has_nxt = it.next(p, hg, tid, nxt.pc);
      if (has_nxt) stage_piece(nxt, p, l);
    };

    // Block stream: the issue cursor (piece 0 = cur, 1 = nxt; block jb) runs up to 3
    // blocks ahead of the block being computed, across the boundary into nxt.
    int ic_piece = 0, ic_j = 0;
    int issued = 0;                              // blocks issued in this unit
    int g0 = 0;                                  // stream index of cur's block 0
    auto issue_next = [&]() {
      if (ic_piece == 0 && ic_j >= cur.nblk) {
        if (!nxt_known || !has_nxt) return;
        ic_piece = 1;
        ic_j = 0;
      }
      if (ic_piece == 0) {
        issue_piece_block<FP8>(cur, p, ic_j, issued, smem, w, l);
      } else {
        if (ic_j >= nxt.nblk) return;
        issue_piece_block<FP8>(nxt, p, ic_j, issued, smem, w, l);
      }
      ++ic_j;
      ++issued;
    };

    // query fragments (B operand): row l16, features 32kk + 8g4 .. +7; padding rows
    // compute with head 0's query and are never stored.  The next piece's query is
    // loaded while the current piece finishes, before its output stores, so that
    // waiting for it does not wait for those stores (vmcnt is in order).
    bf16x8_t qf[18];
    auto load_q = [&](int bq) {
      const uint16_t* qrow = p.q + (int64_t)bq * p.q_sb + (int64_t)tq * p.q_st + (int64_t)(row_ok ? head : 0) * p.q_sh;
#pragma unroll
      for (int kk = 0; kk < 18; ++kk) qf[kk] = *reinterpret_cast<const bf16x8_t*>(qrow + 32 * kk + 8 * g4);
    };
    bool q_ready = false;

    while (true) {
      const int b = cur.pc.b, t_begin = cur.pc.t_begin, t_end = cur.pc.t_end, seq = cur.pc.seq;
      const int nblk = cur.nblk;
      const int nvis = seq - p.q_len + 1 + tq;
      auto valid_of = [&](int j) {
        const int v = t_end - (t_begin + kBlk * j);
        return v < kBlk ? v : kBlk;
      };

      // the piece's first three blocks: in flight already (issued while the previous
      // piece finished) or issued here.  The stream must be three blocks ahead before
      // step 0: each step issues only one more.
      // When nothing of the piece is in flight (a unit's first piece), only block 0 goes
      // out ahead of the query and the rest after it, so that step 0 waits for block 0
      // and the query only.
      const int issued_at_start = issued;
      const bool fresh = !q_ready && issued == g0;
      for (int k = 0; k < (fresh ? 1 : 3) && issued < g0 + 3; ++k) issue_next();
      const bool topped = issued >= g0 + 3;
      const int before_q = issued;
      if (!q_ready) load_q(b);
      fetch_nxt();
      if (!topped) {
        for (int k = 0; k < 3 && issued < g0 + 3; ++k) issue_next();
      }
      // the query and the blocks issued before it (block 0 among them) have landed once
      // at most the operations issued after the query are outstanding: the blocks issued
      // after it, or with the query loaded at the end of the previous piece, at least
      // that piece's 8 output stores per wave
      if (fresh) wait_query_and_block0<FP8>(issued - before_q, w);
      else if (!q_ready || issued != issued_at_start) wait_vmcnt<0>();
      else wait_vmcnt<8>();
#pragma unroll
      for (int kk = 0; kk < 18; ++kk) asm volatile("" ::"v"(qf[kk]));

      f32x4_t o[8];
      float m = -INFINITY, lsum = 0.f, lrsum = 0.f, m_seen = -INFINITY;
      int ovf = 0;
      float m_restart = -INFINITY;
      for (int attempt = 0; attempt < 2; ++attempt) {
#pragma unroll
        for (int f = 0; f < 8; ++f) o[f] = f32x4_t{};
        m = m_restart;
        lsum = 0.f;
        lrsum = 0.f;
        m_seen = -INFINITY;
        ovf = 0;
        if (tid == 0) *ovf_flag = 0;
        if (attempt > 0 && nblk > 0) {
          // drop whatever the stream had in flight and restage this piece from block 0
          load_q(b);
          wait_vmcnt<0>();
          ic_piece = 0;
          ic_j = 0;
          g0 = issued;
          load_page_ids(cur.ids, p, b, cur.pg0, cur.pg1, l);
          issue_next();
          issue_next();
          issue_next();
          wait_vmcnt<0>();
        }
        if constexpr (!FP8) {
          if (nblk == 1) zero_own_tail(smem + (g0 & (kRing - 1)) * kSlot, valid_of(0), w, l);
        }
        lds_barrier();                           // block 0 visible, flag reset published
        if constexpr (FP8) {
          if (nblk > 0) {
            convert_fp8_blk(smem + kRaw + (g0 & (kRing - 1)) * kBlkBytesFp8, smem,
                            reinterpret_cast<MLA_LDS float*>(smem + kFac), valid_of(0), tid, p.scale_log2);
            lds_barrier();
          }
        }

        // Block step: scores of block j and their weights into P(j), with the PV MFMAs
        // of block j-1 between the row maxima and the exponentials (WITH_PV), then the
        // hand-over to block j+1.
        auto step = [&](int j, auto with_pv) {
          constexpr bool WITH_PV = decltype(with_pv)::value;
          const int g = g0 + j;
          const MLA_LDS char* cb = smem + (FP8 ? (j & 1) : (g & (kRing - 1))) * kSlot;
          const MLA_LDS float* fac = reinterpret_cast<const MLA_LDS float*>(smem + kFac + (j & 1) * kFacBytes);
          const int tok0 = t_begin + kBlk * j + 16 * th + 4 * g4;   // token of element 0

          f32x4_t sc = narrow_scores(cb, qf, kbase);
          float mt = -INFINITY;
          {
            f32x4_t kf;
            if constexpr (FP8) kf = *reinterpret_cast<const MLA_LDS f32x4_t*>(fac + 16 * th + 4 * g4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float x = sc[i] * (FP8 ? kf[i] : p.scale_log2);
              x = (tok0 + i < nvis) ? x : -INFINITY;
              sc[i] = x;
              mt = fmaxf(mt, x);
            }
            mt = max_xor32(max_xor16(mt));
          }
          if constexpr (!WITH_PV) {
            if (attempt == 0) {
              // reference max of each row from the piece's first block: the two token
              // halves meet in LDS
              if (w < 2 && g4 == 0) stats[th * kNRows + l16][0] = mt;
              lds_barrier();
              m = fmaxf(stats[l16][0], stats[kNRows + l16][0]);
            }
          }
          m_seen = fmaxf(m_seen, mt);
          const float base = m == -INFINITY ? 0.f : m;
          ovf |= (mt > base + kRefSlack) ? 1 : 0;

          if constexpr (WITH_PV) {
            const int gp = g - 1;
            narrow_pv(smem + (FP8 ? ((j - 1) & 1) : (gp & (kRing - 1))) * kSlot, smem + kNP + ((j - 1) & 1) * kNPBytes,
                      o, vbase, pbase);
          }

          // weights p = 2^(x - m), bf16 for the MFMA (fp8: times v_scale); the sums keep
          // the exact weights (LSE) and the rounded ones (O).  A token whose v_scale is 0
          // has V = 0 and still counts with its rounded weight.
          {
            f32x4_t vf, ivf;
            if constexpr (FP8) {
              vf = *reinterpret_cast<const MLA_LDS f32x4_t*>(fac + kBlk + 16 * th + 4 * g4);
              ivf = *reinterpret_cast<const MLA_LDS f32x4_t*>(fac + 2 * kBlk + 16 * th + 4 * g4);
            }
            bf16x4_t pk;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float pr = __builtin_amdgcn_exp2f(sc[i] - base);
              const __bf16 rr = (__bf16)(FP8 ? pr * vf[i] : pr);
              pk[i] = rr;
              lsum += pr;
              lrsum += FP8 ? (vf[i] != 0.f ? (float)rr * ivf[i] : (float)(__bf16)pr) : (float)rr;
            }
            if (w < 2) *reinterpret_cast<MLA_LDS bf16x4_t*>(smem + kNP + (j & 1) * kNPBytes + pwrite) = pk;
          }

          if (j + 1 < nblk) {
            // this wave's share of block j+1 has landed once only the blocks issued after
            // it (at most block j+2) are outstanding
            wait_blocks_after<FP8>(issued - (g + 2), w);
            if constexpr (!FP8) {
              if (j + 2 == nblk) zero_own_tail(smem + ((g + 1) & (kRing - 1)) * kSlot, valid_of(j + 1), w, l);
            }
          }
          lds_barrier();                         // Y(j)
          issue_next();                          // block g+3 of the stream
          if constexpr (FP8) {
            if (j + 1 < nblk) {
              convert_fp8_blk(smem + kRaw + ((g + 1) & (kRing - 1)) * kBlkBytesFp8, smem + ((j + 1) & 1) * kSlot,
                              reinterpret_cast<MLA_LDS float*>(smem + kFac + ((j + 1) & 1) * kFacBytes),
                              valid_of(j + 1), tid, p.scale_log2);
              lds_barrier();                     // Z(j+1)
            }
          }
        };
        if (nblk > 0) {
          step(0, std::false_type{});
          for (int j = 1; j < nblk; ++j) step(j, std::true_type{});
        }
        // this piece's scores are done: the next piece's query loads go out now (a redo
        // reloads this piece's query)
        q_ready = has_nxt;
        if (has_nxt) load_q(nxt.pc.b);
        if (nblk > 0) {
          const int jl = nblk - 1;
          narrow_pv(smem + (FP8 ? (jl & 1) : ((g0 + jl) & (kRing - 1))) * kSlot, smem + kNP + (jl & 1) * kNPBytes, o,
                    vbase, pbase);
        }
        // any row over the reference slack: the whole workgroup redoes the piece
        if (ovf) *ovf_flag = 1;
        lds_barrier();
        const int redo = *ovf_flag;
        lds_barrier();
        if (redo == 0) break;
        // restart with the largest score seen in either token half of each row
        m_seen = max_xor32(max_xor16(m_seen));
        if (w < 2 && g4 == 0) stats[th * kNRows + l16][0] = m_seen;
        lds_barrier();
        m_restart = fmaxf(stats[l16][0], stats[kNRows + l16][0]);
        lds_barrier();
      }

      // ---- epilogue ----
      // row sums over the 4 lane groups, then over the two token halves
      {
        const float a = sum_xor32(sum_xor16(lsum));
        const float c = sum_xor32(sum_xor16(lrsum));
        if (w < 2 && g4 == 0) stats[th * kNRows + l16] = f32x4_t{m, a, c, 0.f};
      }
      lds_barrier();
      const bool single = cur.pc.nsplit == 1;
      const size_t slot = (size_t)cur.pc.slot * p.n_hg + hg;
      const float lt = stats[l16][1] + stats[kNRows + l16][1];
      const float lr = stats[l16][2] + stats[kNRows + l16][2];
      const float inv = lr > 0.f ? 1.0f / lr : 0.f;
      if (w == 0 && g4 == 0 && row_ok) {
        const float lse_v = lt > 0.f ? (m + __builtin_log2f(lt)) * kLn2 : -INFINITY;
        if (single) p.lse[((int64_t)b * p.q_len + tq) * p.N + head] = lse_v;
        else p.part_lse[slot * kNRows + l16] = lse_v;
      }
      // this lane's accumulators: row l16, features 128w + 16f + 4g4 .. +3
      if (row_ok) {
        if (single) {
          uint16_t* orow = p.out + (int64_t)b * p.o_sb + (int64_t)tq * p.o_st + (int64_t)head * p.o_sh + 128 * w + 4 * g4;
#pragma unroll
          for (int f = 0; f < 8; ++f) {
            const bf16x4_t v = {(__bf16)(o[f][0] * inv), (__bf16)(o[f][1] * inv), (__bf16)(o[f][2] * inv),
                                (__bf16)(o[f][3] * inv)};
            *reinterpret_cast<bf16x4_t*>(orow + 16 * f) = v;
          }
        } else {
          float* prow = p.part_o + (slot * kNRows + l16) * kLatent + 128 * w + 4 * g4;
#pragma unroll
          for (int f = 0; f < 8; ++f) *reinterpret_cast<f32x4_t*>(prow + 16 * f) = o[f] * inv;
        }
      }
      lds_barrier();                             // stats and P free for the next piece

      fetch_nxt();
      if (!has_nxt) break;
      // the next piece becomes current; its blocks continue the stream
      g0 += nblk;
      cur = nxt;
      nxt_known = false;
      if (ic_piece == 1) {
        ic_piece = 0;                            // the cursor was already inside it
      } else {
        ic_j = 0;                                // nothing of it issued yet
      }
    }
    wait_vmcnt<0>();                             // nothing in flight into LDS at the unit's end
  }
}

// ---------------------------------------------------------------------------
// Wide variant: 64 query rows per unit, 8 waves in two roles, 32-token blocks
// ---------------------------------------------------------------------------
// Division of labour inside a workgroup (w = wave; waves w and w + 4 share a SIMD, so
// every SIMD runs one wave of each role):
//  * score waves (w = 0..3): wave w owns query rows 32*(w >> 1) .. +31 and tokens
//    16*(w & 1) .. +15 of each block.  S^T = K . Q^T runs on 16x16x32 MFMA: one K
//    fragment (16 tokens x 32 features, from LDS) feeds two MFMAs (row halves), the
//    wave's query rows stay in registers (B operand, 144 registers).  The softmax runs
//    here too; the bf16 weights P go to LDS.
//  * value waves (w = 4..7, v = w - 4): wave v owns latent features 128v .. 128v+127 of
//    all 64 rows.  O^T += V^T . P^T runs on 32x32x16 MFMA, V^T from LDS transpose reads
//    of the same staged rows (the latent is V), P^T read back from LDS; the wave's O is
//    128 accumulator registers.  These waves also issue the block copies.
// The roles form a two-stage pipeline: while the score waves compute block j, the value
// waves accumulate block j-1, so on every SIMD one wave's LDS reads, softmax and waits
// run under the other's MFMAs.  Every staged K byte is read by two waves, every V byte
// by one.  Per block (one barrier Y(j) for all eight waves):
//    score waves:  QK(j) -> softmax(j) -> P(j) to LDS                                  -> Y(j)
//    value waves:  PV(j-1) with the copy of block j+2 spread over it -> wait for own
//                  copy of block j+1                                                   -> Y(j)
// A copy instruction holds its wave while the CU's memory pipeline takes it, so each
// wave's share goes out in three smaller bursts between MFMAs.  Blocks j+1 and j+2 are in
// flight while block j is computed.  bf16 blocks land in a
// 4-slot ring; fp8 blocks land raw in a 4-slot ring and are read in place (codes
// converted to bf16 in registers, exactly).  Each role's loop is its own code region, so
// a wave's registers hold only its role's state.
constexpr int kWWaves = 8;
constexpr int kWRows = 64;                             // query rows per wide unit
constexpr int kWP = kStageEnd;                         // P: 2 buffers x 64 rows x 64 B
constexpr int kWPBytes = kWRows * 64;
constexpr int kWStats = kWP + 2 * kWPBytes;            // per token half and row {m, l, lr, -}
constexpr int kWFlag = kWStats + 2 * kWRows * 16;      // overflow flag of the reference max
constexpr int kWPlan = kWFlag + 16;                    // split-plan scratch
constexpr int kWLdsBytes = kWPlan + kPlanLdsBytes;
constexpr int kWStagePitch32 = 272;                    // epilogue staging: 64 fp32 of a row + pad
constexpr int kWStagePitch16 = 144;                    // 64 bf16 of a row + pad
constexpr int kWStageBytes = 32 * kWStagePitch32;      // per value wave
static_assert(4 * kWStageBytes <= kSlot, "epilogue staging fits one block slot");
static_assert(kWLdsBytes <= 160 * 1024, "LDS budget");

// S^T = K . Q^T of this wave's 16 tokens of a block for its 32 rows: 18 steps of 32
// features, each one K fragment read (kPrefK steps ahead, a rolling register buffer)
// and two 16x16x32 MFMAs (row halves rs = 0, 1).
__device__ __forceinline__ void wide_scores(const MLA_LDS char* blk, const bf16x8_t (&qf)[2][18],
                                            const uint32_t (&kbase)[2], f32x4_t (&sc)[2]) {
  constexpr int kPrefK = 4;
  uint32_t ka[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) ka[m] = opaque(lds_addr(blk) + kbase[m]);
  bf16x8_t kbuf[kPrefK];
#pragma unroll
  for (int d = 0; d < kPrefK; ++d) kbuf[d] = lds_read_b128_at(ka[d & 1] + (d >> 1) * kBlkGroupBytes);
  __builtin_amdgcn_sched_group_barrier(0x100, kPrefK, 0);
  sc[0] = f32x4_t{};
  sc[1] = f32x4_t{};
#pragma unroll
  for (int kk = 0; kk < 18; ++kk) {
    const bf16x8_t a = kbuf[kk % kPrefK];
    const int nk = kk + kPrefK;
    if (nk < 18) kbuf[kk % kPrefK] = lds_read_b128_at(ka[nk & 1] + (nk >> 1) * kBlkGroupBytes);
    sc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[0][kk], sc[0], 0, 0, 0);
    sc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[1][kk], sc[1], 0, 0, 0);
    if (nk < 18) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  }
}

// O^T[this wave's 128 features][64 rows] += V^T . P^T over one block (2 steps of 16
// tokens).  Step s: V^T fragment of feature block fb = two transpose reads (tokens
// 16s + 8hh + 4r + 0..3, r = 0/1, hh = lane >> 5), P^T fragment of row block rb = one
// 16-byte read of tokens 16s + 8hh .. +7 of row 32rb + (lane & 31).
// Operands of one PV step (V^T fragments via transpose reads, P^T rows), requested
// in two token halves so that the loads can be issued ahead of the MFMAs.
struct WidePvOps {
  uint32_t va_addr[2][2], pa[2];
  bf16x8_t pb[2][2];
  bf16x4_t lo[2][4], hi[2][4];
  __device__ __forceinline__ void init(const MLA_LDS char* blk, const MLA_LDS char* pbuf, const uint32_t (&vbase)[2][2],
                                       const uint32_t (&pbase)[2]) {
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int f1 = 0; f1 < 2; ++f1) va_addr[r][f1] = opaque(lds_addr(blk) + vbase[r][f1]);
#pragma unroll
    for (int s = 0; s < 2; ++s) pa[s] = opaque(lds_addr(pbuf) + pbase[s]);
  }
  __device__ __forceinline__ void load(int s) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) pb[s][rb] = lds_read_b128_at(pa[s] + rb * 2048);
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) {
      const uint32_t off = (uint32_t)((fb >> 1) * kBlkGroupBytes + s * 2048);
      lo[s][fb] = lds_read_tr16_at(va_addr[0][fb & 1] + off);
      hi[s][fb] = lds_read_tr16_at(va_addr[1][fb & 1] + off);
    }
  }
};

// Work placed between a PV's MFMAs: mid() after the first token half's, end() after the
// last (the value waves issue parts of the next block's copy there).
struct NoHook {
  __device__ __forceinline__ void mid() const {}
  __device__ __forceinline__ void end() const {}
};

// O^T += V^T . P^T for one block.  The first token half's operands were requested by
// the caller (ops.load(0)); the second half's are requested while the first half's
// MFMAs run.
template <class Hook = NoHook>
__device__ __forceinline__ void wide_pv_mfma(WidePvOps& ops, f32x16_t (&o)[4][2], const Hook& hook = Hook{}) {
  __builtin_amdgcn_sched_group_barrier(0x100, 10, 0);
  ops.load(1);
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) {
      const bf16x8_t va = {ops.lo[s][fb][0], ops.lo[s][fb][1], ops.lo[s][fb][2], ops.lo[s][fb][3],
                           ops.hi[s][fb][0], ops.hi[s][fb][1], ops.hi[s][fb][2], ops.hi[s][fb][3]};
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        o[fb][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, ops.pb[s][rb], o[fb][rb], 0, 0, 0);
        if (s == 0) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (fb * 2 + rb < 5) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
      }
    }
    if (s == 0) hook.mid();
  }
  hook.end();
}

template <class Hook = NoHook>
__device__ __forceinline__ void wide_pv(const MLA_LDS char* blk, const MLA_LDS char* pbuf,
                                        f32x16_t (&o)[4][2], const uint32_t (&vbase)[2][2],
                                        const uint32_t (&pbase)[2], const Hook& hook = Hook{}) {
  WidePvOps ops;
  ops.init(blk, pbuf, vbase, pbase);
  ops.load(0);
  wide_pv_mfma(ops, o, hook);
}

// ---- fp8 rows read in place (wide variant) ----
// The raw block keeps the cache's row layout: token t at t * 584 (576 e4m3 codes, then
// k_scale and v_scale).  Fragments are converted to bf16 in registers (exact).
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(u32x2_t c) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c[0], 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c[0], 1.0f, true);
  const bf16x2_t e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c[1], 1.0f, false);
  const bf16x2_t f = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c[1], 1.0f, true);
  return bf16x8_t{a[0], a[1], b[0], b[1], e[0], e[1], f[0], f[1]};
}

__device__ __forceinline__ u32x2_t lds_read_b64_at(uint32_t addr) {
  return *reinterpret_cast<const MLA_LDS u32x2_t*>((uintptr_t)addr);
}

// Transpose read of 8-bit data: the 16 lanes of a group each give 8 bytes; lane pair
// (2k, 2k+1) forms row k of an 8 x 16 byte matrix and lane i receives column i.
__device__ __forceinline__ u32x2_t lds_read_tr8_at(uint32_t addr) {
  const v2i32_t r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(reinterpret_cast<MLA_LDS v2i32_t*>((uintptr_t)addr));
  return u32x2_t{(uint32_t)r[0], (uint32_t)r[1]};
}

// S^T of this wave's 16 tokens for its 32 rows from raw fp8 codes: 18 steps of 32
// features, each one 8-byte code read (kPrefK steps ahead) converted to bf16.
__device__ __forceinline__ void wide_scores_fp8(const MLA_LDS char* blk, const bf16x8_t (&qf)[2][18], uint32_t kbase8,
                                                f32x4_t (&sc)[2]) {
  constexpr int kPrefK = 3;                              // timed against 2, 4, 6, 9
  const uint32_t ka = opaque(lds_addr(blk) + kbase8);
  u32x2_t kbuf[kPrefK];
#pragma unroll
  for (int d = 0; d < kPrefK; ++d) kbuf[d] = lds_read_b64_at(ka + 32 * d);
  sc[0] = f32x4_t{};
  sc[1] = f32x4_t{};
#pragma unroll
  for (int kk = 0; kk < 18; ++kk) {
    const bf16x8_t a = fp8x8_to_bf16(kbuf[kk % kPrefK]);
    const int nk = kk + kPrefK;
    if (nk < 18) kbuf[kk % kPrefK] = lds_read_b64_at(ka + 32 * nk);
    sc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[0][kk], sc[0], 0, 0, 0);
    sc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[1][kk], sc[1], 0, 0, 0);
  }
}

// O^T += V^T . P^T over one raw fp8 block: per step of 16 tokens and feature block fb,
// one 8-bit transpose read gives each lane its feature's 8 tokens.
template <class Hook = NoHook>
__device__ __forceinline__ void wide_pv_fp8(const MLA_LDS char* blk, const MLA_LDS char* pbuf, f32x16_t (&o)[4][2],
                                            uint32_t vbase8, const uint32_t (&pbase)[2], const Hook& hook = Hook{}) {
  const uint32_t va = opaque(lds_addr(blk) + vbase8);
  uint32_t pa[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) pa[s] = opaque(lds_addr(pbuf) + pbase[s]);
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    bf16x8_t pb[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) pb[rb] = lds_read_b128_at(pa[s] + rb * 2048);
    u32x2_t vc[4];
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) vc[fb] = lds_read_tr8_at(va + s * 16 * kRowBytesFp8 + 32 * fb);
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) {
      const bf16x8_t a = fp8x8_to_bf16(vc[fb]);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        o[fb][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[rb], o[fb][rb], 0, 0, 0);
    }
    if (s == 0) hook.mid();
  }
  hook.end();
}

// Bytes of rows >= valid inside this wave's share of a raw fp8 block (flat 16-byte
// chunks 64k + lane, k = w + 4i) become zero: codes and scales past the end of a
// sequence may hold NaN patterns.  Row ends are multiples of 8 bytes.
__device__ __forceinline__ void zero_own_tail_fp8(MLA_LDS char* blk, int valid, int w, int l) {
  const int end = valid * kRowBytesFp8;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int o = 16 * (64 * (w + 4 * i) + l);
    if (o + 16 <= kBlkBytesFp8 && o + 16 > end) {
      if (o >= end) *reinterpret_cast<MLA_LDS u32x4_t*>(blk + o) = u32x4_t{0u, 0u, 0u, 0u};
      else *reinterpret_cast<MLA_LDS u32x2_t*>(blk + o + 8) = u32x2_t{0u, 0u};
    }
  }
}

// wait until the block issued `later` blocks before the newest one has landed
// (value waves: per-wave instruction counts of a block 9 bf16; 5, 5, 5, 4 fp8)
template <bool FP8>
__device__ __forceinline__ void wait_block_before(int later, int v) {
  if (later <= 0) wait_vmcnt<0>();
  else if (later == 1) wait_blocks_after<FP8>(1, v);
  else wait_query_and_block0<FP8>(2, v);
}

// One value wave's share of a block copy, looked up ahead of its instructions: the half
// page in the cache and the wave's LDS destination in the ring slot.
struct BlockCopy {
  const char* src;
  uint32_t lds;
};

template <bool FP8>
__device__ __forceinline__ BlockCopy prepare_copy(StagedPiece& sp, const DecodeParams& p, int jb, int g,
                                                  MLA_LDS char* smem, int v, int l) {
  jb = __builtin_amdgcn_readfirstlane(jb);
  g = __builtin_amdgcn_readfirstlane(g);
  const char* pg = page_ptr(sp.ids, p, sp.pc.b, sp.pg0 + (jb >> 1), sp.pg1, l, FP8);
  BlockCopy c;
  if constexpr (FP8) {
    c.src = pg + (jb & 1) * kBlkBytesFp8;
    c.lds = lds_addr(smem + kRaw + (g & (kRing - 1)) * kBlkBytesFp8) + 1024u * (uint32_t)v;
  } else {
    c.src = pg + (jb & 1) * kBlkBytesBf16;
    c.lds = lds_addr(smem + (g & (kRing - 1)) * kSlot) + 1024u * (uint32_t)v;
  }
  return c;
}

// Instruction I of the wave's share (the split of issue_blk_bf16 / issue_blk_fp8: bf16
// instruction I = tokens 8v .. 8v+7 of 128-byte column I, I < 9; fp8 instruction I = flat
// chunks 64(v + 4I) + lane, I < 5, while inside the block).  voff: the lane's offset in
// that split (bf16: token row and swizzled chunk; fp8: 1024v + 16 lane).
template <bool FP8, int I>
__device__ __forceinline__ void copy_insn(const BlockCopy& c, uint32_t voff, int v, int l) {
  // (the LDS base is wave-uniform; readfirstlane states it to the compiler)
  const uint32_t lds = __builtin_amdgcn_readfirstlane(c.lds);
  if constexpr (FP8) {
    if constexpr (I < 5) {
      if ((v + 4 * I) * 64 + l < kBlkChunksFp8) dma_16B<0, 4096 * I>(c.src + 4096 * I, voff, lds);
    }
  } else {
    if constexpr (I < 9) dma_16B<128 * I, kBlkGroupBytes * I>(c.src, voff, lds);
  }
}

// Instructions [B, E) of the share, issued only when the copy exists (`on`, uniform)
template <bool FP8, int B, int E>
__device__ __forceinline__ void copy_part(const BlockCopy& c, bool on, uint32_t voff, int v, int l) {
  if constexpr (B < E) {
    if (on) copy_insn<FP8, B>(c, voff, v, l);
    copy_part<FP8, B + 1, E>(c, on, voff, v, l);
  }
}

// A block copy spread over a PV: one third before it (begin), one after its first token
// half (mid), the rest after it (end), so that the copy instructions, which hold their
// wave while the CU's memory pipeline takes them, go out in smaller bursts.
template <bool FP8>
struct SpreadCopy {
  static constexpr int kN = FP8 ? 5 : 9;
  static constexpr int kA = (kN + 2) / 3, kB = 2 * (kN + 2) / 3;
  const BlockCopy& c;
  bool on;
  uint32_t voff;
  int v, l;
  __device__ __forceinline__ void begin() const { copy_part<FP8, 0, kA>(c, on, voff, v, l); }
  __device__ __forceinline__ void mid() const { copy_part<FP8, kA, kB>(c, on, voff, v, l); }
  __device__ __forceinline__ void end() const { copy_part<FP8, kB, kN>(c, on, voff, v, l); }
};

// ---- a unit's first query through LDS ----
// At a unit's first piece the 64 query rows (73,728 B) are copied once into LDS by all
// eight waves and both token-half score waves of a row group read them from there, so
// the start-up burst carries each query byte once instead of twice.  Row R sits at
// R * 1152 with its 16-byte chunk c at position c ^ qswz(R), qswz taking row bits 1, 2
// and 3: the 8-lane groups a ds_read_b128 may serve together (equal lane bits {0, 1, 4},
// or 8 or 16 consecutive lanes) each hit distinct bank groups; on the GPU this took the
// staging's conflict cycles from 3.7e5 to 1.2e5 per call with bits 2, 3 only.  Region: ring slots 2
// and 3 for bf16 rows (block 2 is issued once the query has been read), the unused
// converted slots for fp8 rows.
constexpr int kQRowBytes = kRow * 2;                   // 1152
constexpr int kQLdsBytes = kWRows * kQRowBytes;        // 73728
static_assert(kQLdsBytes <= 2 * kSlot && 2 * kSlot + kQLdsBytes <= kStageEnd, "query staging LDS plan");

__device__ __forceinline__ int qswz(int R) { return (((R >> 2) & 1) << 2) | (((R >> 1) & 1) << 1) | ((R >> 3) & 1); }

// the query rows' byte offsets from request b's query fit 32 bits (uniform)
__device__ __forceinline__ bool query_lds_fits(const DecodeParams& p) {
  const int64_t hi = ((int64_t)(p.q_len - 1) * p.q_st + (int64_t)(p.N - 1) * p.q_sh) * 2 + kQRowBytes;
  return p.q_st >= 0 && p.q_sh >= 0 && hi < (int64_t)0x7fffffff;
}

template <int I>
__device__ __forceinline__ void query_dma_one(const DecodeParams& p, const uint16_t* base, int hg, uint32_t lds, int w,
                                              int l) {
  const int e = 64 * (w + 8 * I) + l;                  // LDS chunk of this lane
  const int R = e / 72;
  const int col = (e - 72 * R) ^ qswz(R);
  const int hl = R / p.q_len, tq = R - hl * p.q_len;
  int head = hg * p.hg_heads + hl;
  head = head < p.N ? head : 0;                        // padding rows: head 0 (never stored)
  const uint32_t voff = (uint32_t)(((int64_t)tq * p.q_st + (int64_t)head * p.q_sh) * 2 + col * 16);
  dma_16B<0, 8192 * I>(base, voff, lds);
}

template <int... I>
__device__ __forceinline__ void query_dma_seq(std::integer_sequence<int, I...>, const DecodeParams& p,
                                              const uint16_t* base, int hg, uint32_t lds, int w, int l) {
  (query_dma_one<I>(p, base, hg, lds, w, l), ...);
}

// The same copy through registers, for query strides whose row offsets need 64 bits
__device__ __forceinline__ void stage_query_lds_wide_strides(const DecodeParams& p, int b, int hg, MLA_LDS char* qs,
                                                             int w, int l) {
#pragma unroll 1
  for (int i = 0; i < 9; ++i) {
    const int e = 64 * (w + 8 * i) + l;
    const int R = e / 72;
    const int col = (e - 72 * R) ^ qswz(R);
    const int hl = R / p.q_len, tq = R - hl * p.q_len;
    int head = hg * p.hg_heads + hl;
    head = head < p.N ? head : 0;
    const uint16_t* src = p.q + (int64_t)b * p.q_sb + (int64_t)tq * p.q_st + (int64_t)head * p.q_sh + 8 * col;
    *reinterpret_cast<MLA_LDS u32x4_t*>(qs + 16 * e) = *reinterpret_cast<const u32x4_t*>(src);
  }
}

// wave w's share (9 instructions) of the copy of request b's 64 query rows of head group hg
__device__ __forceinline__ void stage_query_lds(const DecodeParams& p, int b, int hg, MLA_LDS char* qs, int w, int l) {
  b = __builtin_amdgcn_readfirstlane(b);
  hg = __builtin_amdgcn_readfirstlane(hg);
  const uint16_t* base = p.q + (int64_t)b * p.q_sb;
  query_dma_seq(std::make_integer_sequence<int, 9>{}, p, base, hg, lds_addr(qs) + 1024u * (uint32_t)w, w, l);
}

// The role that issues the block copies (and waits for them before each hand-over).
constexpr bool kCopyByScore = false;
// Blocks of the stream issued ahead of the one being computed (at most kRing - 1).
constexpr int kWDepth = 3;
static_assert(kWDepth >= 2 && kWDepth < kRing, "copy depth");

// One role's walk over the workgroup's units (QK: score waves, else value waves).  Both
// roles run the same sequence of barriers and plan lookups.
template <bool FP8, bool P64, bool QK>
__device__ __forceinline__ void wide_role(const DecodeParams& p, MLA_LDS char* smem, MLA_LDS long long* plan_lds,
                                          const PlanTotals<P64>& tot, int seq0, int tid, int w, int l) {
  constexpr bool COPY = QK == kCopyByScore;     // this role issues the block copies
  const int l16 = l & 15, g4 = l >> 4;
  const int rg = (w >> 1) & 1, th = w & 1;      // score waves: row group, token half
  const int v = w & 3;                          // value waves: feature quarter and DMA share
  MLA_LDS int* ovf_flag = reinterpret_cast<MLA_LDS int*>(smem + kWFlag);
  MLA_LDS f32x4_t* stats = reinterpret_cast<MLA_LDS f32x4_t*>(smem + kWStats);   // [2][64]

  // Per-lane LDS offsets, fixed for the whole kernel.
  // K fragment of step kk: token 16*th + l16, chunk 4kk + g4 (group kk >> 1, in-group
  // chunk 4(kk & 1) + g4).
  uint32_t kbase[2];
  {
    const int t = 16 * th + l16;
#pragma unroll
    for (int m = 0; m < 2; ++m) kbase[m] = (uint32_t)(t * 8 + ((4 * m + g4) ^ page_swz(t))) * 16;
  }
  // V^T transpose reads: the 16-lane group g4 reads tokens 16s + 8*(l >> 5) + 4r + (l16 >> 2)
  // at features 128v + 32fb + 16(g4 & 1) + 4(l16 & 3); chunk 16v + 4fb + 2(g4 & 1) +
  // ((l16 >> 1) & 1) lies in group 2v + (fb >> 1) at in-group chunk
  // 4(fb & 1) + 2(g4 & 1) + ((l16 >> 1) & 1).  s and fb >> 1 only add offsets.
  uint32_t vbase[2][2];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int f1 = 0; f1 < 2; ++f1) {
      const int t = 8 * (l >> 5) + 4 * r + (l16 >> 2);
      const int cin = 4 * f1 + 2 * (g4 & 1) + ((l16 >> 1) & 1);
      vbase[r][f1] = (uint32_t)(2 * v * kBlkGroupBytes + (t * 8 + (cin ^ page_swz(t))) * 16 + 8 * (l16 & 1));
    }
  // P rows: 64 B = 4 chunks of 8 tokens; chunk a of row R sits at position a ^ ((R >> 2) & 3)
  // and row R at p_row(R), so that the 8-lane groups of a 16-byte read (rows with equal
  // bits 0, 1, both chunks of a lane pair) hit 8 distinct bank groups.
  // fp8 (raw rows): K codes of token 16th + l16 at features 32kk + 8g4; the 8-bit
  // transpose read of step s and feature block fb: lane pair (2k, 2k+1) of group g4 gives
  // token 16s + 8(g4 >> 1) + k, features 128v + 32fb + 16(g4 & 1) + 8(l16 & 1) .. +7.
  const uint32_t kbase8 = (uint32_t)((16 * th + l16) * kRowBytesFp8 + 8 * g4);
  const uint32_t vbase8 =
      (uint32_t)((8 * (g4 >> 1) + (l16 >> 1)) * kRowBytesFp8 + 128 * v + 16 * (g4 & 1) + 8 * (l16 & 1));
  uint32_t pbase[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int R = l & 31;
    pbase[s] = (uint32_t)(p_row(R) * 64 + (((2 * s + (l >> 5)) ^ ((R >> 2) & 3)) * 16));
  }
  // copying waves: this lane's offset in the wave's share of a block copy
  uint32_t copy_voff;
  if constexpr (FP8) {
    copy_voff = (uint32_t)(1024 * v + 16 * l);
  } else {
    const int t = 8 * v + (l >> 3);
    copy_voff = (uint32_t)(t * kRowBytesBf16 + ((l & 7) ^ page_swz(t)) * 16);
  }

  for (int u = blockIdx.x; u < p.n_units; u += gridDim.x) {
    int sid, hg;
    unit_to_stream(u, p.n_hg, &sid, &hg);
    if (sid >= p.n_streams) continue;
    PieceIter<P64> it;
    it.init(p, plan_lds, tot, sid, tid, seq0);
    StagedPiece cur, nxt;
    if (!it.next(p, hg, tid, cur.pc)) continue;
    stage_piece(cur, p, l);
    // the following piece is looked up once the current one's first blocks are in flight
    bool nxt_known = false, has_nxt = false;
    auto fetch_nxt = [&]() {
      if (nxt_known) return;
      nxt_known = true;
      has_nxt = it.next(p, hg, tid, nxt.pc);
      if (has_nxt) stage_piece(nxt, p, l);
    };
    // Block stream (as in the narrow variant): the issue cursor (piece 0 = cur, 1 = nxt;
    // block jb) runs up to 3 blocks ahead of the block being computed, across the
    // boundary into nxt.  Both roles keep the cursor; the value waves issue the copies.
    int ic_piece = 0, ic_j = 0;
    int issued = 0;                              // blocks issued in this unit
    int landed = 0;                              // value waves: blocks [0, landed) waited for
    int g0 = 0;                                  // stream index of cur's block 0
    // the cursor's next block: false when nothing is left to issue; the copying role
    // also gets the block's copy (its instructions are issued by the caller)
    auto next_copy = [&](BlockCopy& c) -> bool {
      if (ic_piece == 0 && ic_j >= cur.nblk) {
        if (!nxt_known || !has_nxt) return false;
        ic_piece = 1;
        ic_j = 0;
      }
      if (ic_piece == 0) {
        if constexpr (COPY) c = prepare_copy<FP8>(cur, p, ic_j, issued, smem, v, l);
      } else {
        if (ic_j >= nxt.nblk) return false;
        if constexpr (COPY) c = prepare_copy<FP8>(nxt, p, ic_j, issued, smem, v, l);
      }
      ++ic_j;
      ++issued;
      return true;
    };
    auto issue_next = [&]() {
      BlockCopy c;
      const bool on = next_copy(c);
      if constexpr (COPY) copy_part<FP8, 0, FP8 ? 5 : 9>(c, on, copy_voff, v, l);
    };

    // score waves: the two query rows this lane owns, 32rg + 16rs + l16
    bool row_ok[2];
    int qhead[2], qtq[2];
#pragma unroll
    for (int rs = 0; rs < 2; ++rs) {
      const int r = 32 * rg + 16 * rs + l16;
      const int hl = r / p.q_len, tq = r - hl * p.q_len;
      qhead[rs] = hg * p.hg_heads + hl;
      qtq[rs] = tq;
      row_ok[rs] = qhead[rs] < p.N;
    }
    // query fragments (B operand of the 16x16x32 MFMA): row 32rg + 16rs + l16, features
    // 32kk + 8*g4 .. +7.  Padding rows (head >= N) compute with head 0's query; their
    // results are never stored.  (Nothing may read the loaded registers before they are
    // needed: a select on them would make the compiler wait for the loads right here.)
    bf16x8_t qf[QK ? 2 : 1][QK ? 18 : 1];
    auto load_q = [&](int bq) {
      if constexpr (QK) {
#pragma unroll
        for (int rs = 0; rs < 2; ++rs) {
          const uint16_t* qrow = p.q + (int64_t)bq * p.q_sb + (int64_t)qtq[rs] * p.q_st +
                                 (int64_t)(row_ok[rs] ? qhead[rs] : 0) * p.q_sh;
#pragma unroll
          for (int kk = 0; kk < 18; ++kk) qf[rs][kk] = *reinterpret_cast<const bf16x8_t*>(qrow + 32 * kk + 8 * g4);
        }
      }
    };
    // the next piece's query is loaded at the end of the current piece's scores
    bool q_ready = false;

    while (true) {
      const int b = cur.pc.b, t_begin = cur.pc.t_begin, t_end = cur.pc.t_end, seq = cur.pc.seq;
      const int nsplit = cur.pc.nsplit, pslot = cur.pc.slot;
      const int nblk = cur.nblk;
      int nvis[2];
#pragma unroll
      for (int rs = 0; rs < 2; ++rs) nvis[rs] = seq - p.q_len + 1 + qtq[rs];

      auto valid_of = [&](int j) {
        const int vv = t_end - (t_begin + kBlk * j);
        return vv < kBlk ? vv : kBlk;
      };
      // the piece's first three blocks: in flight already (issued while the previous
      // piece finished) or issued here
      if (issued == 0 && p.q_len == 1) {
        // the unit's first piece with one query row per head: block 0, the query (once,
        // into LDS), block 1 (fp8: and block 2); the copying waves' wait leaves only the
        // later blocks in flight.  (With two query rows per head the staging measured no
        // faster than loading the query twice, so those batches keep the direct loads.)
        MLA_LDS char* qs = smem + (FP8 ? 0 : 2 * kSlot);
        // lane-dependent addresses from an opaque lane id: hoisted out of the unit loop
        // they would stay live across it
        const int lq = (int)opaque((uint32_t)l);
        issue_next();
        const int before_q = issued;             // blocks issued before the query copy
        if (query_lds_fits(p)) stage_query_lds(p, b, hg, qs, w, lq);
        else stage_query_lds_wide_strides(p, b, hg, qs, w, lq);
        issue_next();
        if constexpr (FP8) issue_next();
        // (a short piece has fewer blocks: only those issued after the query may stay out)
        if constexpr (COPY) wait_query_and_block0<FP8>(issued - before_q, v);
        else wait_vmcnt<0>();
        lds_barrier();
        if constexpr (QK) {
          // chunk (4kk + g4) ^ qswz(R) = 4 (kk ^ s2) + (g4 ^ s01), s2 / s01: bit 2 / bits 0-1 of
          // qswz(R); R and R + 16 share qswz, so one base per parity of kk serves both rows
          const int R = 32 * rg + (lq & 15);
          const int sw = qswz(R);
          const uint32_t a0 = lds_addr(qs) + (uint32_t)(R * kQRowBytes + 16 * ((lq >> 4) ^ (sw & 3)));
          const uint32_t ae = opaque(a0 + 64u * (uint32_t)(sw >> 2));   // even kk
          const uint32_t ao = opaque(a0 - 64u * (uint32_t)(sw >> 2));   // odd kk
#pragma unroll
          for (int rs = 0; rs < 2; ++rs)
#pragma unroll
            for (int kk = 0; kk < 18; ++kk)
              qf[rs][kk] = lds_read_b128_at(((kk & 1) ? ao : ae) + (uint32_t)(rs * 16 * kQRowBytes + 64 * kk));
        }
        lds_barrier();                           // the query region is free again
        if constexpr (!FP8) issue_next();        // block 2, into ring slot 2
      } else {
        for (int k = 0; k < kWDepth && issued < g0 + kWDepth; ++k) issue_next();
        if constexpr (QK) {
          if (!q_ready) load_q(b);
        }
      }
      fetch_nxt();
      if constexpr (COPY) {
        // block 0 of the piece: waited for at the end of the previous piece, or now (an
        // empty piece has no block 0: stream block g0 belongs to a later piece and may not
        // be issued yet)
        if (nblk > 0 && landed <= g0) {
          wait_block_before<FP8>(issued - (g0 + 1), v);
          landed = g0 + 1;
        }
      }
      if constexpr (QK) {
        // the compiler waits for the query loads here
#pragma unroll
        for (int rs = 0; rs < 2; ++rs)
#pragma unroll
          for (int kk = 0; kk < 18; ++kk) asm volatile("" ::"v"(qf[rs][kk]));
      }

      f32x16_t o[QK ? 1 : 4][QK ? 1 : 2];
      // score waves, per row half: reference max m and base (m, or 0 while m = -inf), the
      // weight sums, and this lane's largest y = x - base so far
      float m[2], base[2], lsum[2], lrsum[2], ym[2];
      int ovf = 0;
      float m_restart[2] = {-INFINITY, -INFINITY};
      for (int attempt = 0; attempt < 2; ++attempt) {
        if constexpr (!QK) {
#pragma unroll
          for (int fb = 0; fb < 4; ++fb)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) o[fb][rb] = f32x16_t{};
        }
#pragma unroll
        for (int rs = 0; rs < 2; ++rs) {
          m[rs] = m_restart[rs];
          base[rs] = m[rs] == -INFINITY ? 0.f : m[rs];
          lsum[rs] = 0.f;
          lrsum[rs] = 0.f;
          ym[rs] = -INFINITY;
        }
        ovf = 0;
        if (tid == 0) *ovf_flag = 0;
        if (attempt > 0 && nblk > 0) {
          // drop whatever the stream had in flight and restage this piece from block 0
          load_q(b);
          wait_vmcnt<0>();
          ic_piece = 0;
          ic_j = 0;
          g0 = issued;
          if constexpr (COPY) load_page_ids(cur.ids, p, b, cur.pg0, cur.pg1, l);
          for (int k = 0; k < kWDepth; ++k) issue_next();
          wait_vmcnt<0>();
          landed = issued;
        }
        if constexpr (COPY) {
          if (nblk == 1) {
            if constexpr (FP8) zero_own_tail_fp8(smem + kRaw + (g0 & (kRing - 1)) * kBlkBytesFp8, valid_of(0), v, l);
            else zero_own_tail(smem + (g0 & (kRing - 1)) * kSlot, valid_of(0), v, l);
          }
        }
        lds_barrier();                           // block 0 visible, flag reset published

        // Block step j: the score waves compute the weights P(j), the value waves the PV
        // of block j-1; then the hand-over to block j+1.
        auto step = [&](int j) {
          const int g = g0 + j;
          if constexpr (QK) {
            if (j > 0) {
              BlockCopy c;
              next_copy(c);                           // the cursor moves as in the value waves
            }
            const MLA_LDS char* cb =
                FP8 ? smem + kRaw + (g & (kRing - 1)) * kBlkBytesFp8 : smem + (g & (kRing - 1)) * kSlot;
            const int tok0 = t_begin + kBlk * j + 16 * th + 4 * g4;   // token of this lane's element 0
            f32x4_t sc[2];
            // fp8: {k_scale, v_scale} of this lane's 4 tokens, read from the raw rows
            f32x2_t kv[4];
            if constexpr (FP8) {
#pragma unroll
              for (int i = 0; i < 4; ++i)
                kv[i] = *reinterpret_cast<const MLA_LDS f32x2_t*>(cb + (16 * th + 4 * g4 + i) * kRowBytesFp8 + kRow);
              wide_scores_fp8(cb, qf, kbase8, sc);
            } else {
              wide_scores(cb, qf, kbase, sc);
            }
            // scores -> log2 domain relative to the reference: y = x - base with x = score *
            // scale * log2 e (fp8: times k_scale), -inf where the causal / length mask hides the
            // token.  Element i of row half rs is token tok0 + i.
            f32x4_t kf;
#pragma unroll
            for (int i = 0; i < 4; ++i) kf[i] = FP8 ? kv[i][0] * p.scale_log2 : p.scale_log2;
            float y[2][4];
            if (j == 0 && attempt == 0) {
              // reference max of each row from the unit's first block: the two token halves
              // of a row live in two waves, so their maxima meet in LDS
              float mt[2];
#pragma unroll
              for (int rs = 0; rs < 2; ++rs) {
                mt[rs] = -INFINITY;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  float x = sc[rs][i] * kf[i];
                  x = (tok0 + i < nvis[rs]) ? x : -INFINITY;
                  y[rs][i] = x;
                  mt[rs] = fmaxf(mt[rs], x);
                }
                mt[rs] = max_xor32(max_xor16(mt[rs]));
              }
              if (g4 == 0) {
#pragma unroll
                for (int rs = 0; rs < 2; ++rs) stats[th * kWRows + 32 * rg + 16 * rs + l16][0] = mt[rs];
              }
              lds_barrier();
#pragma unroll
              for (int rs = 0; rs < 2; ++rs) {
                const int R = 32 * rg + 16 * rs + l16;
                m[rs] = fmaxf(stats[R][0], stats[kWRows + R][0]);
                base[rs] = m[rs] == -INFINITY ? 0.f : m[rs];
#pragma unroll
                for (int i = 0; i < 4; ++i) y[rs][i] -= base[rs];
              }
            } else {
#pragma unroll
              for (int rs = 0; rs < 2; ++rs)
#pragma unroll
                for (int i = 0; i < 4; ++i) y[rs][i] = __builtin_fmaf(sc[rs][i], kf[i], -base[rs]);
              // the mask only matters where the block reaches past the shortest visible length
              if (t_begin + kBlk * (j + 1) > seq - p.q_len + 1) {
#pragma unroll
                for (int rs = 0; rs < 2; ++rs)
#pragma unroll
                  for (int i = 0; i < 4; ++i)
                    if (tok0 + i >= nvis[rs]) y[rs][i] = -INFINITY;
              }
            }
            // this lane's largest y of each row: the slack check and the restart reference
            // (maximum: no canonicalising moves; y is never NaN for finite inputs)
#pragma unroll
            for (int rs = 0; rs < 2; ++rs) {
              const float bm = __builtin_elementwise_maximum(__builtin_elementwise_maximum(y[rs][0], y[rs][1]),
                                                             __builtin_elementwise_maximum(y[rs][2], y[rs][3]));
              ym[rs] = __builtin_elementwise_maximum(ym[rs], bm);
              ovf |= (bm > kRefSlack) ? 1 : 0;
            }
            // weights: p = 2^y, rounded to bf16 for the MFMA (fp8: times v_scale); the sums
            // keep both the exact weights (LSE) and the rounded ones (O).  A token whose
            // v_scale is 0 has V = 0 and still counts with its rounded weight.
            f32x4_t vf, ivf;
            if constexpr (FP8) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                vf[i] = kv[i][1];
                // hardware reciprocal (1 ulp): only normalises the weight sum
                ivf[i] = kv[i][1] != 0.f ? __builtin_amdgcn_rcpf(kv[i][1]) : 0.f;
              }
            }
            MLA_LDS char* pw = smem + kWP + (j & 1) * kWPBytes;
#pragma unroll
            for (int rs = 0; rs < 2; ++rs) {
              bf16x4_t pk;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float pr = __builtin_amdgcn_exp2f(y[rs][i]);
                const __bf16 rr = (__bf16)(FP8 ? pr * vf[i] : pr);
                pk[i] = rr;
                lsum[rs] += pr;
                if constexpr (FP8) lrsum[rs] += vf[i] != 0.f ? (float)rr * ivf[i] : (float)(__bf16)pr;
              }
              if constexpr (!FP8) {
                // sum of the rounded weights, two at a time
                const bf16x2_t one2 = {(__bf16)1.0f, (__bf16)1.0f};
                lrsum[rs] = __builtin_amdgcn_fdot2_f32_bf16(bf16x2_t{pk[0], pk[1]}, one2, lrsum[rs], false);
                lrsum[rs] = __builtin_amdgcn_fdot2_f32_bf16(bf16x2_t{pk[2], pk[3]}, one2, lrsum[rs], false);
              }
              // row R, tokens 16th + 4g4 .. +3: chunk 2th + (g4 >> 1), half g4 & 1
              const int R = 32 * rg + 16 * rs + l16;
              const int a = 2 * th + (g4 >> 1);
              *reinterpret_cast<MLA_LDS bf16x4_t*>(pw + p_row(R) * 64 + ((a ^ ((R >> 2) & 3)) * 16) + 8 * (g4 & 1)) =
                  pk;
            }
          } else {
            if (j == 0 && attempt == 0) lds_barrier();   // the score waves' reference-max exchange
            if (j > 0) {
              // PV of block j-1, with the copy of stream block g+2 spread over it
              BlockCopy c;
              const bool on = next_copy(c);
              const SpreadCopy<FP8> cp{c, on, copy_voff, v, l};
              cp.begin();
              const MLA_LDS char* pbuf = smem + kWP + ((j - 1) & 1) * kWPBytes;
              if constexpr (FP8)
                wide_pv_fp8(smem + kRaw + ((g - 1) & (kRing - 1)) * kBlkBytesFp8, pbuf, o, vbase8, pbase, cp);
              else
                wide_pv(smem + ((g - 1) & (kRing - 1)) * kSlot, pbuf, o, vbase, pbase, cp);
            }
          }
          if constexpr (COPY) {
            // this wave's share of stream block g+1 (this piece's or the next one's) has
            // landed once only the blocks issued after it (at most g+2) are outstanding
            if (issued > g + 1) {
              wait_blocks_after<FP8>(issued - (g + 2), v);
              landed = g + 2;
              if (j + 2 == nblk) {
                if constexpr (FP8)
                  zero_own_tail_fp8(smem + kRaw + ((g + 1) & (kRing - 1)) * kBlkBytesFp8, valid_of(j + 1), v, l);
                else
                  zero_own_tail(smem + ((g + 1) & (kRing - 1)) * kSlot, valid_of(j + 1), v, l);
              }
            }
          }
          lds_barrier();                              // Y(j)
        };
        for (int j = 0; j < nblk; ++j) step(j);
        if constexpr (QK) {
          if (nblk > 0) {
            BlockCopy c;
            next_copy(c);
          }
          // This piece's scores are done: the next piece's query loads go out now (a redo
          // reloads this piece's query).
          q_ready = has_nxt;
          if (has_nxt) load_q(nxt.pc.b);
        } else {
          if (nblk > 0) {
            // the last block's PV, with the copy of stream block g0 + nblk + kWDepth - 1
            const int jl = nblk - 1;
            BlockCopy c;
            const bool on = next_copy(c);
            const SpreadCopy<FP8> cp{c, on, copy_voff, v, l};
            cp.begin();
            const MLA_LDS char* pbuf = smem + kWP + (jl & 1) * kWPBytes;
            if constexpr (FP8)
              wide_pv_fp8(smem + kRaw + ((g0 + jl) & (kRing - 1)) * kBlkBytesFp8, pbuf, o, vbase8, pbase, cp);
            else
              wide_pv(smem + ((g0 + jl) & (kRing - 1)) * kSlot, pbuf, o, vbase, pbase, cp);
          }
        }
        // any row over the reference slack: the whole workgroup redoes the piece
        if (ovf) *ovf_flag = 1;
        lds_barrier();
        const int redo = *ovf_flag;
        lds_barrier();
        if (redo == 0) break;
        // restart with the largest score seen in either token half of each row
        if constexpr (QK) {
          float m_seen[2];
#pragma unroll
          for (int rs = 0; rs < 2; ++rs) m_seen[rs] = max_xor32(max_xor16(ym[rs] + base[rs]));
          if (g4 == 0) {
#pragma unroll
            for (int rs = 0; rs < 2; ++rs) stats[th * kWRows + 32 * rg + 16 * rs + l16][0] = m_seen[rs];
          }
        }
        lds_barrier();
        if constexpr (QK) {
#pragma unroll
          for (int rs = 0; rs < 2; ++rs) {
            const int R = 32 * rg + 16 * rs + l16;
            m_restart[rs] = fmaxf(stats[R][0], stats[kWRows + R][0]);
          }
        }
        lds_barrier();
      }

      // ---- epilogue ----
      // lane-dependent addresses below derive from an opaque copy of the lane id, so
      // the compiler cannot hoist them out of the piece loop (they would stay live
      // across the whole block loop)
      const int le = (int)opaque((uint32_t)l);
      const size_t slot = (size_t)pslot * p.n_hg + hg;
      const bool single = nsplit == 1;
      // row sums: over the 4 lane groups of a score wave, then over the two token halves
      if constexpr (QK) {
#pragma unroll
        for (int rs = 0; rs < 2; ++rs) {
          const float a = sum_xor32(sum_xor16(lsum[rs]));
          const float c = sum_xor32(sum_xor16(lrsum[rs]));
          if (g4 == 0) stats[th * kWRows + 32 * rg + 16 * rs + l16] = f32x4_t{m[rs], a, c, 0.f};
        }
      }
      lds_barrier();
      if constexpr (QK) {
        if (th == 0 && g4 == 0) {
#pragma unroll
          for (int rs = 0; rs < 2; ++rs) {
            const int R = 32 * rg + 16 * rs + l16;
            const float lt = stats[R][1] + stats[kWRows + R][1];
            const float lse_v = lt > 0.f ? (m[rs] + __builtin_log2f(lt)) * kLn2 : -INFINITY;
            if (row_ok[rs]) {
              if (single) p.lse[((int64_t)b * p.q_len + qtq[rs]) * p.N + qhead[rs]] = lse_v;
              else p.part_lse[slot * p.m_wg + R] = lse_v;
            }
          }
        }
      } else {
        // This lane's accumulators: row 32rb + (l & 31), features 128v + 32fb + 8i +
        // 4(l >> 5) + 0..3.  They are staged, half a row block at a time, through this
        // wave's part of the one ring slot the next piece's blocks leave free (the slot of
        // this piece's last block; fp8: the unused first slot) and stored as whole row
        // segments (256 B fp32, 128 B bf16 per row and wave).
        MLA_LDS char* stage = smem + (FP8 ? 0 : ((g0 + nblk + 3) & (kRing - 1)) * kSlot) + v * kWStageBytes;
        const int c32 = le & 31, h32 = le >> 5;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const int R = 32 * rb + c32;
          const float lr_row = stats[R][2] + stats[kWRows + R][2];
          const float inv = lr_row > 0.f ? 1.0f / lr_row : 0.f;
#pragma unroll
          for (int fh = 0; fh < 2; ++fh) {
            if (single) {
#pragma unroll
              for (int fl = 0; fl < 2; ++fl)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const int fb = 2 * fh + fl;
                  const bf16x4_t vv = {(__bf16)(o[fb][rb][4 * i] * inv), (__bf16)(o[fb][rb][4 * i + 1] * inv),
                                       (__bf16)(o[fb][rb][4 * i + 2] * inv), (__bf16)(o[fb][rb][4 * i + 3] * inv)};
                  *reinterpret_cast<MLA_LDS bf16x4_t*>(stage + c32 * kWStagePitch16 + (32 * fl + 8 * i + 4 * h32) * 2) =
                      vv;
                }
              asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
              // all reads first: the global stores may alias LDS as far as the compiler knows,
              // so interleaving would serialise every read behind the previous store
              u32x4_t vr[4];
#pragma unroll
              for (int k = 0; k < 4; ++k)
                vr[k] = *reinterpret_cast<const MLA_LDS u32x4_t*>(stage + (8 * k + (le >> 3)) * kWStagePitch16 +
                                                                  (le & 7) * 16);
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                const int Rr = 32 * rb + 8 * k + (le >> 3);
                const int hl_r = Rr / p.q_len, tq_r = Rr - hl_r * p.q_len;
                const int head_r = hg * p.hg_heads + hl_r;
                if (head_r < p.N) {
                  uint16_t* orow = p.out + (int64_t)b * p.o_sb + (int64_t)tq_r * p.o_st + (int64_t)head_r * p.o_sh;
                  *reinterpret_cast<u32x4_t*>(orow + 128 * v + 64 * fh + 8 * (le & 7)) = vr[k];
                }
              }
            } else {
#pragma unroll
              for (int fl = 0; fl < 2; ++fl)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const int fb = 2 * fh + fl;
                  const f32x4_t vv = {o[fb][rb][4 * i] * inv, o[fb][rb][4 * i + 1] * inv, o[fb][rb][4 * i + 2] * inv,
                                      o[fb][rb][4 * i + 3] * inv};
                  *reinterpret_cast<MLA_LDS f32x4_t*>(stage + c32 * kWStagePitch32 + (32 * fl + 8 * i + 4 * h32) * 4) =
                      vv;
                }
              asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
              for (int kb = 0; kb < 2; ++kb) {
                u32x4_t vr[4];
#pragma unroll
                for (int k = 0; k < 4; ++k)
                  vr[k] = *reinterpret_cast<const MLA_LDS u32x4_t*>(stage + (4 * (4 * kb + k) + (le >> 4)) * kWStagePitch32 +
                                                                    (le & 15) * 16);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                  float* prow = p.part_o + (slot * p.m_wg + 32 * rb + 4 * (4 * kb + k) + (le >> 4)) * kLatent + 128 * v +
                                64 * fh + 4 * (le & 15);
                  *reinterpret_cast<u32x4_t*>(prow) = vr[k];
                }
              }
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // stage reads done before reuse
          }
        }
      }
      lds_barrier();                             // stats and P free for the next piece

      fetch_nxt();
      if (!has_nxt) break;
      // the next piece becomes current; its blocks continue the stream
      g0 += nblk;
      cur = nxt;
      nxt_known = false;
      if (ic_piece == 1) {
        ic_piece = 0;                            // the cursor was already inside it
      } else {
        ic_j = 0;                                // nothing of it issued yet
      }
    }
    wait_vmcnt<0>();                             // nothing in flight into LDS at the unit's end
  }
}

template <bool FP8, bool P64>
__global__ __launch_bounds__(kWWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_wide_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[kWLdsBytes];
  MLA_LDS char* smem = (MLA_LDS char*)(smem_raw);
  const int tid = threadIdx.x;
  const int w = wave_id();
  const int l = lane_id();
  MLA_LDS long long* plan_lds = reinterpret_cast<MLA_LDS long long*>(smem + kWPlan);
  PlanTotals<P64> tot{1, 1};
  int seq0 = 0;
  if (p.num_splits == 0) tot = plan_prefix<P64>(p, plan_lds, tid, &seq0);
  if (w < 4) wide_role<FP8, P64, true>(p, smem, plan_lds, tot, seq0, tid, w, l);
  else wide_role<FP8, P64, false>(p, smem, plan_lds, tot, seq0, tid, w, l);
}


// ---------------------------------------------------------------------------
// Split merge ([vLLM-MLA] §Prefill merge of partial states; §Triton MLA second stage):
// o = sum_s w_s o_s / sum_s w_s with w_s = exp(lse_s - max_s lse_s), lse = max + ln sum w.
// grid = (B * n_hg, m_wg / 4), 4 waves: one query row per wave, 8 features per lane;
// the partial rows and LSEs of up to 8 splits are in flight together.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void merge_kernel(DecodeParams p) {
  const int b = blockIdx.x / p.n_hg;
  const int hg = blockIdx.x - b * p.n_hg;
  const int4 rq = p.req[b];
  const int first = rq.x, nsplit = rq.y;
  if (nsplit <= 1) return;
  // the decode kernel writes req[b] with slots inside the workspace; checked anyway so
  // that no read can leave it
  if (first < 0 || nsplit > p.max_slots || first > p.max_slots - nsplit) return;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int r = blockIdx.y * 4 + w;
  if (r >= p.m_wg) return;
  const int hl = r / p.q_len, tq = r - hl * p.q_len;
  const int head = hg * p.hg_heads + hl;
  if (head >= p.N) return;
  // Splits are taken 8 at a time: the 8 partial rows and their LSEs are loaded
  // together (every lane reads the same LSE values), then folded into a running
  // (max, weight sum, weighted sum) with the usual rescale when the max grows.
  float M = -INFINITY;
  f32x4_t a0 = {}, a1 = {};
  float wsum = 0.f;
  // KS splits per round (4 when a request has at most 4: no clamped duplicate loads)
  auto fold = [&](auto ks_c) {
    constexpr int KS = decltype(ks_c)::value;
    for (int s0 = 0; s0 < nsplit; s0 += KS) {
      f32x4_t v[KS][2];
      float ls[KS];
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const int s = s0 + k < nsplit ? s0 + k : nsplit - 1;        // clamp: in bounds, weight 0 below
        const size_t slot = (size_t)(first + s) * p.n_hg + hg;
        const f32x4_t* src = reinterpret_cast<const f32x4_t*>(p.part_o + (slot * p.m_wg + r) * kLatent + 8 * l);
        v[k][0] = src[0];
        v[k][1] = src[1];
        ls[k] = s0 + k < nsplit ? p.part_lse[slot * p.m_wg + r] : -INFINITY;
      }
      float mc = M;
#pragma unroll
      for (int k = 0; k < KS; ++k) mc = fmaxf(mc, ls[k]);
      if (mc == -INFINITY) continue;                                 // all splits so far empty
      const float resc = M == -INFINITY ? 0.f : __expf(M - mc);
      wsum *= resc;
      a0 *= resc;
      a1 *= resc;
      M = mc;
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const float wt = ls[k] == -INFINITY ? 0.f : __expf(ls[k] - M);
        wsum += wt;
        a0 += wt * v[k][0];
        a1 += wt * v[k][1];
      }
    }
  };
  if (nsplit <= 4) fold(std::integral_constant<int, 4>{});
  else fold(std::integral_constant<int, 8>{});
  const float Mb = M == -INFINITY ? 0.f : M;
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  uint16_t* orow = p.out + (int64_t)b * p.o_sb + (int64_t)tq * p.o_st + (int64_t)head * p.o_sh + 8 * l;
  const bf16x8_t v = {(__bf16)(a0[0] * inv), (__bf16)(a0[1] * inv), (__bf16)(a0[2] * inv),
                      (__bf16)(a0[3] * inv), (__bf16)(a1[0] * inv), (__bf16)(a1[1] * inv),
                      (__bf16)(a1[2] * inv), (__bf16)(a1[3] * inv)};
  *reinterpret_cast<bf16x8_t*>(orow) = v;
  if (l == 0) p.lse[((int64_t)b * p.q_len + tq) * p.N + head] = wsum > 0.f ? Mb + __logf(wsum) : -INFINITY;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
struct Shape {
  bool wide;
  int m_wg, hg_heads, n_hg, max_slots;
};

inline bool decode_shape(int32_t B, int32_t q_len, int32_t N, int32_t num_splits, Shape* s) {
  if (B < 1 || (q_len != 1 && q_len != 2) || N < 1 || N > MLA_MAX_HEADS) return false;
  if (num_splits < 0 || num_splits > 4096) return false;
  s->wide = q_len * N > 16;
  s->m_wg = s->wide ? kWRows : 16;
  s->hg_heads = s->m_wg / q_len;
  s->n_hg = (N + s->hg_heads - 1) / s->hg_heads;
  int64_t mp;
  if (num_splits == 0) mp = (int64_t)B + MLA_AUTO_MAX_EXTRA_PAIRS;
  else mp = (int64_t)B * num_splits;
  mp += 8;
  if (mp > (1 << 24)) return false;
  s->max_slots = (int)mp;
  return true;
}

struct WsLayout {
  size_t req, part_lse, part_o, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline WsLayout ws_layout(int32_t B, const Shape& s) {
  WsLayout w;
  size_t off = 0;
  w.req = off;
  off = align256(off + (size_t)B * sizeof(int4));
  const size_t rows = (size_t)s.max_slots * s.n_hg * s.m_wg;
  w.part_lse = off;
  off = align256(off + rows * sizeof(float));
  w.part_o = off;
  off = align256(off + rows * kLatent * sizeof(float));
  w.total = off;
  return w;
}


// Streams of the plan: in automatic mode one per workgroup and head group, so every
// unit runs concurrently, with a multiple of 8 streams when there are several head
// groups (sibling order); forced mode: B * num_splits.
inline int64_t plan_streams(const Shape& s, int32_t num_splits, int32_t B, const DeviceInfo& di) {
  const int64_t cus = ((int64_t)di.cu_count + 7) / 8 * 8;
  if (num_splits != 0) return (int64_t)B * num_splits;
  int64_t streams = s.n_hg == 1 ? cus : cus / (8 * s.n_hg) * 8;
  if (streams < 8) streams = 8;
  if (streams > MLA_AUTO_MAX_EXTRA_PAIRS) streams = MLA_AUTO_MAX_EXTRA_PAIRS;
  return streams;
}

// Launches the decode kernels (and the merge) for filled-in parameters: the plan's
// stream and unit counts, the 32/64-bit plan variant, the kernel variant.
static mla_status_t decode_launch(DecodeParams p, const Shape& s, int32_t kv_dtype, int32_t num_splits,
                                  int32_t B, int32_t max_pages_per_seq, const DeviceInfo& di,
                                  hipStream_t hs) {
  // One workgroup (512 threads wide, 256 narrow; most of the LDS) per CU.  Automatic plan: one
  // stream per workgroup and head group, so every unit runs concurrently; with
  // several head groups the stream count is a multiple of 8 (sibling order).
  const int64_t cus = ((int64_t)di.cu_count + 7) / 8 * 8;
  const int64_t streams = plan_streams(s, num_splits, B, di);
  const int64_t units = s.n_hg == 1 ? streams : (streams + 7) / 8 * 8 * s.n_hg;
  if (units > (int64_t)1 << 30) return MLA_ERR_SHAPE;
  p.n_streams = (int32_t)streams;
  p.n_units = (int32_t)units;
  int64_t grid = cus < units ? cus : units;
  if (grid < 1) grid = 1;

  // The automatic plan's products fit in 32 bits when total * (streams + 1) and
  // len * pages do (total <= B * (overhead + block-table width), len <= overhead + width);
  // only batches beyond that bound run the kernels with 64-bit plan arithmetic.
  const uint64_t stretch = (uint64_t)kSegOverhead + (uint64_t)max_pages_per_seq;
  const bool p64 = num_splits == 0 && ((uint64_t)B * stretch > 0xFFFFFFFFull / (uint64_t)(streams + 1) ||
                                       stretch * (uint64_t)max_pages_per_seq > 0xFFFFFFFFull);
  const dim3 g((unsigned)grid), blk(s.wide ? kWWaves * 64 : 256);
  if (kv_dtype == MLA_KV_BF16) {
    if (p64) {
      if (s.wide) hipLaunchKernelGGL((decode_wide_kernel<false, true>), g, blk, 0, hs, p);
      else hipLaunchKernelGGL((decode_narrow_kernel<false, true>), g, blk, 0, hs, p);
    } else {
      if (s.wide) hipLaunchKernelGGL((decode_wide_kernel<false, false>), g, blk, 0, hs, p);
      else hipLaunchKernelGGL((decode_narrow_kernel<false, false>), g, blk, 0, hs, p);
    }
  } else {
    if (p64) {
      if (s.wide) hipLaunchKernelGGL((decode_wide_kernel<true, true>), g, blk, 0, hs, p);
      else hipLaunchKernelGGL((decode_narrow_kernel<true, true>), g, blk, 0, hs, p);
    } else {
      if (s.wide) hipLaunchKernelGGL((decode_wide_kernel<true, false>), g, blk, 0, hs, p);
      else hipLaunchKernelGGL((decode_narrow_kernel<true, false>), g, blk, 0, hs, p);
    }
  }
  if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;
  if (num_splits != 1) {
    dim3 mg((unsigned)(B * s.n_hg), (unsigned)((s.m_wg + 3) / 4));
    hipLaunchKernelGGL(merge_kernel, mg, dim3(256), 0, hs, p);
  }
  return launch_status();
}
}  // namespace mla

extern "C" size_t mla_decode_workspace_size(int32_t B, int32_t q_len, int32_t N, int32_t num_splits) {
  mla::Shape s;
  if (!mla::decode_shape(B, q_len, N, num_splits, &s)) return 0;
  return mla::ws_layout(B, s).total;
}

namespace mla {

// Argument checks of mla_decode and mla_decode_noalloc (everything but the workspace)
inline mla_status_t decode_check(const void* q, int64_t q_stride_b, int64_t q_stride_t, int64_t q_stride_h,
                                 const void* kv_cache, int32_t kv_dtype, int64_t num_pages,
                                 const int32_t* block_table, int64_t bt_stride_b, int32_t max_pages_per_seq,
                                 const int32_t* seq_lens, int32_t B, int32_t q_len, int32_t N,
                                 float softmax_scale, int32_t num_splits, const void* out, int64_t o_stride_b,
                                 int64_t o_stride_t, int64_t o_stride_h, const float* lse, Shape* s) {
  if (kv_dtype != MLA_KV_BF16 && kv_dtype != MLA_KV_FP8_E4M3) return MLA_ERR_DTYPE;
  if (!decode_shape(B, q_len, N, num_splits, s)) return MLA_ERR_SHAPE;
  if (num_pages < 1 || max_pages_per_seq < 1 || bt_stride_b < max_pages_per_seq) return MLA_ERR_SHAPE;
  if (!(softmax_scale > 0.f) || !__builtin_isfinite(softmax_scale)) return MLA_ERR_SHAPE;
  if (!q || !kv_cache || !block_table || !seq_lens || !out || !lse) return MLA_ERR_NULL;
  if (!aligned16(q) || !aligned16(kv_cache) || !aligned16(out) || !mult8(q_stride_b) || !mult8(q_stride_t) ||
      !mult8(q_stride_h) || !mult8(o_stride_b) || !mult8(o_stride_t) || !mult8(o_stride_h) ||
      (reinterpret_cast<uintptr_t>(block_table) & 3u) != 0 || (reinterpret_cast<uintptr_t>(seq_lens) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
    return MLA_ERR_ALIGN;
  return MLA_OK;
}

// Parameters of one decode call whose workspace is `ws` laid out as `wl` with
// `max_slots` partial slots
inline DecodeParams decode_params(const void* q, int64_t q_stride_b, int64_t q_stride_t, int64_t q_stride_h,
                                  const void* kv_cache, int64_t num_pages, const int32_t* block_table,
                                  int64_t bt_stride_b, int32_t max_pages_per_seq, const int32_t* seq_lens,
                                  int32_t B, int32_t q_len, int32_t N, float softmax_scale, int32_t num_splits,
                                  char* ws, const WsLayout& wl, int32_t max_slots, const Shape& s, void* out,
                                  int64_t o_stride_b, int64_t o_stride_t, int64_t o_stride_h, float* lse) {
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
  p.req = reinterpret_cast<int4*>(ws + wl.req);
  p.part_lse = reinterpret_cast<float*>(ws + wl.part_lse);
  p.part_o = reinterpret_cast<float*>(ws + wl.part_o);
  p.num_splits = num_splits;
  p.max_slots = max_slots;
  return p;
}

}  // namespace mla

extern "C" mla_status_t mla_decode(const void* q, int64_t q_stride_b, int64_t q_stride_t,
                                   int64_t q_stride_h, const void* kv_cache, int32_t kv_dtype,
                                   int64_t num_pages, const int32_t* block_table, int64_t bt_stride_b,
                                   int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t B,
                                   int32_t q_len, int32_t N, float softmax_scale, int32_t num_splits,
                                   void* workspace, size_t workspace_bytes, void* out,
                                   int64_t o_stride_b, int64_t o_stride_t, int64_t o_stride_h,
                                   float* lse, void* stream) {
  using namespace mla;
  Shape s;
  mla_status_t st = decode_check(q, q_stride_b, q_stride_t, q_stride_h, kv_cache, kv_dtype, num_pages, block_table,
                                 bt_stride_b, max_pages_per_seq, seq_lens, B, q_len, N, softmax_scale, num_splits,
                                 out, o_stride_b, o_stride_t, o_stride_h, lse, &s);
  if (st != MLA_OK) return st;
  if (!workspace) return MLA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return MLA_ERR_ALIGN;
  const WsLayout wl = ws_layout(B, s);
  if (workspace_bytes < wl.total) return MLA_ERR_WORKSPACE;
  DeviceInfo di;
  st = device_info(&di);
  if (st != MLA_OK) return st;
  // a seq_len is an int32, so no request reaches past page 2^25 - 1: wider tables are
  // read only that far (this also keeps the kernels' page * 64 arithmetic in 32 bits)
  if (max_pages_per_seq > kMaxPagesPerSeq) max_pages_per_seq = kMaxPagesPerSeq;
  const DecodeParams p = decode_params(q, q_stride_b, q_stride_t, q_stride_h, kv_cache, num_pages, block_table,
                                       bt_stride_b, max_pages_per_seq, seq_lens, B, q_len, N, softmax_scale,
                                       num_splits, static_cast<char*>(workspace), wl, s.max_slots, s, out,
                                       o_stride_b, o_stride_t, o_stride_h, lse);
  return decode_launch(p, s, kv_dtype, num_splits, B, max_pages_per_seq, di,
                       reinterpret_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------
// Decode without a caller workspace, for callers that cannot allocate: the split
// table and partials live in one file-scope device array per GPU.
// ---------------------------------------------------------------------------
namespace mla {

static __device__ __align__(256) char scratch[MLA_DECODE_SCRATCH_BYTES];

// This GPU's address of `scratch`, looked up once per device with that device current
// (in host code the array's name is only a host-side handle, not a device address)
inline mla_status_t scratch_ptr(char** out) {
  constexpr int kMaxDev = 64;
  static std::atomic<int> state[kMaxDev];   // 0 = not looked up, 1 = ptrs[dev] valid
  static char* ptrs[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return MLA_ERR_HIP;
  if (state[dev].load(std::memory_order_acquire) == 0) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return MLA_ERR_HIP;
    ptrs[dev] = static_cast<char*>(ptr);     // every racing thread stores the same value
    state[dev].store(1, std::memory_order_release);
  }
  *out = ptrs[dev];
  return MLA_OK;
}

// Workspace layout with exactly the partial slots this device's plan can use: automatic
// mode B + streams (+ the 8 spare of decode_shape), forced mode B * num_splits (+ 8);
// num_splits == 1 writes no partials, so only the request table is laid out.
inline WsLayout ws_layout_exact(int32_t B, const Shape& s, int32_t num_splits, int64_t streams,
                                int32_t* max_slots) {
  WsLayout w;
  w.req = 0;
  size_t off = align256((size_t)B * sizeof(int4));
  const int64_t slots = num_splits == 1 ? 0 : (num_splits == 0 ? (int64_t)B + streams + 8 : s.max_slots);
  *max_slots = (int32_t)slots;
  const size_t rows = (size_t)slots * s.n_hg * s.m_wg;
  w.part_lse = off;
  off = align256(off + rows * sizeof(float));
  w.part_o = off;
  off = align256(off + rows * kLatent * sizeof(float));
  w.total = off;
  return w;
}

}  // namespace mla

extern "C" mla_status_t mla_decode_noalloc(const void* q, int64_t q_stride_b, int64_t q_stride_t,
                                           int64_t q_stride_h, const void* kv_cache, int32_t kv_dtype,
                                           int64_t num_pages, const int32_t* block_table, int64_t bt_stride_b,
                                           int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t B,
                                           int32_t q_len, int32_t N, float softmax_scale, int32_t num_splits,
                                           void* out, int64_t o_stride_b, int64_t o_stride_t,
                                           int64_t o_stride_h, float* lse, void* stream) {
  using namespace mla;
  Shape s;
  mla_status_t st = decode_check(q, q_stride_b, q_stride_t, q_stride_h, kv_cache, kv_dtype, num_pages, block_table,
                                 bt_stride_b, max_pages_per_seq, seq_lens, B, q_len, N, softmax_scale, num_splits,
                                 out, o_stride_b, o_stride_t, o_stride_h, lse, &s);
  if (st != MLA_OK) return st;
  DeviceInfo di;
  st = device_info(&di);
  if (st != MLA_OK) return st;
  int32_t max_slots = 0;
  const WsLayout wl = ws_layout_exact(B, s, num_splits, plan_streams(s, num_splits, B, di), &max_slots);
  if (wl.total > (size_t)MLA_DECODE_SCRATCH_BYTES) return MLA_ERR_WORKSPACE;
  char* ws = nullptr;
  st = scratch_ptr(&ws);
  if (st != MLA_OK) return st;
  if (max_pages_per_seq > kMaxPagesPerSeq) max_pages_per_seq = kMaxPagesPerSeq;
  const DecodeParams p = decode_params(q, q_stride_b, q_stride_t, q_stride_h, kv_cache, num_pages, block_table,
                                       bt_stride_b, max_pages_per_seq, seq_lens, B, q_len, N, softmax_scale,
                                       num_splits, ws, wl, max_slots, s, out, o_stride_b, o_stride_t, o_stride_h,
                                       lse);
  return decode_launch(p, s, kv_dtype, num_splits, B, max_pages_per_seq, di,
                       reinterpret_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------
// Variable query lengths ([vLLM-MLA] §投机解码 and §Metadata, QueryLenSupport
// VARLEN: a verification batch mixes requests with 1, 2, 3 ... query tokens;
// causal blocks give row t of a q_len-token block seq_len - q_len + 1 + t visible
// tokens, non-causal draft blocks give every row all of them).  Each query row
// becomes a one-row request with its own length and a copy of its request's
// block-table row (in the workspace), and runs through the same decode kernels.
// ---------------------------------------------------------------------------
namespace mla {

struct VarlenLayout {
  size_t decode, seq, bt, total;
};

inline VarlenLayout varlen_layout(int64_t T, const Shape& s, int32_t max_pages) {
  VarlenLayout v;
  v.decode = 0;
  size_t off = ws_layout((int32_t)T, s).total;
  v.seq = off;
  off = align256(off + (size_t)T * sizeof(int32_t));
  v.bt = off;
  off = align256(off + (size_t)T * (size_t)max_pages * sizeof(int32_t));
  v.total = off;
  return v;
}

// Row r of the flat query: its request (binary search of query_start_loc), its
// visible length, and its request's block-table entries up to that length.
__global__ __launch_bounds__(256) void varlen_expand_kernel(const int32_t* __restrict__ qsl,
                                                            const int32_t* __restrict__ seq_lens, int32_t B,
                                                            int64_t T, int32_t causal,
                                                            const int32_t* __restrict__ bt, int64_t bt_sb,
                                                            int32_t max_pages, int32_t* __restrict__ seq_out,
                                                            int32_t* __restrict__ bt_out) {
  const int64_t r = blockIdx.x;
  if (r >= T) return;
  // largest b with qsl[b] <= r (qsl non-decreasing, qsl[0] = 0)
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (qsl[mid] <= r) lo = mid;
    else hi = mid - 1;
  }
  const int b = lo;
  const int64_t r0 = qsl[b], r1 = qsl[b + 1];
  int seq = 0;
  if (r >= r0 && r < r1) {
    const int64_t s = seq_lens[b] < 0 ? 0 : seq_lens[b];
    const int64_t n = causal ? s - (r1 - r0) + 1 + (r - r0) : s;
    const int64_t cap = (int64_t)max_pages * kPage;
    seq = (int)(n < 0 ? 0 : (n > cap ? cap : n));
  }
  if (threadIdx.x == 0) seq_out[r] = seq;
  const int pages = (seq + kPage - 1) / kPage;
  for (int pg = threadIdx.x; pg < pages; pg += 256) bt_out[r * max_pages + pg] = bt[(int64_t)b * bt_sb + pg];
}

}  // namespace mla

extern "C" size_t mla_decode_varlen_workspace_size(int64_t T, int32_t N, int32_t num_splits,
                                                   int32_t max_pages_per_seq) {
  mla::Shape s;
  if (T < 1 || T > (1 << 24) || max_pages_per_seq < 1) return 0;
  if (max_pages_per_seq > mla::kMaxPagesPerSeq) max_pages_per_seq = mla::kMaxPagesPerSeq;
  if (!mla::decode_shape((int32_t)T, 1, N, num_splits, &s)) return 0;
  return mla::varlen_layout(T, s, max_pages_per_seq).total;
}

extern "C" mla_status_t mla_decode_varlen(const void* q, int64_t q_stride_t, int64_t q_stride_h,
                                          const void* kv_cache, int32_t kv_dtype, int64_t num_pages,
                                          const int32_t* block_table, int64_t bt_stride_b,
                                          int32_t max_pages_per_seq, const int32_t* query_start_loc,
                                          const int32_t* seq_lens, int32_t B, int64_t T, int32_t N,
                                          int32_t causal, float softmax_scale, int32_t num_splits,
                                          void* workspace, size_t workspace_bytes, void* out,
                                          int64_t o_stride_t, int64_t o_stride_h, float* lse, void* stream) {
  using namespace mla;
  if (kv_dtype != MLA_KV_BF16 && kv_dtype != MLA_KV_FP8_E4M3) return MLA_ERR_DTYPE;
  if (T < 1 || T > (1 << 24) || B < 1) return MLA_ERR_SHAPE;
  Shape s;
  if (!decode_shape((int32_t)T, 1, N, num_splits, &s)) return MLA_ERR_SHAPE;
  if (num_pages < 1 || max_pages_per_seq < 1 || bt_stride_b < max_pages_per_seq) return MLA_ERR_SHAPE;
  if (!(softmax_scale > 0.f) || !__builtin_isfinite(softmax_scale)) return MLA_ERR_SHAPE;
  if (!q || !kv_cache || !block_table || !query_start_loc || !seq_lens || !out || !lse) return MLA_ERR_NULL;
  if (!workspace) return MLA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(kv_cache) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 || !mult8(q_stride_t) || !mult8(q_stride_h) ||
      !mult8(o_stride_t) || !mult8(o_stride_h) || (reinterpret_cast<uintptr_t>(block_table) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(query_start_loc) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3u) != 0 || (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
    return MLA_ERR_ALIGN;
  if (max_pages_per_seq > kMaxPagesPerSeq) max_pages_per_seq = kMaxPagesPerSeq;
  const VarlenLayout vl = varlen_layout(T, s, max_pages_per_seq);
  if (workspace_bytes < vl.total) return MLA_ERR_WORKSPACE;
  DeviceInfo di;
  mla_status_t st = device_info(&di);
  if (st != MLA_OK) return st;

  char* ws = static_cast<char*>(workspace);
  int32_t* seq_x = reinterpret_cast<int32_t*>(ws + vl.seq);
  int32_t* bt_x = reinterpret_cast<int32_t*>(ws + vl.bt);
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(varlen_expand_kernel, dim3((unsigned)T), dim3(256), 0, hs, query_start_loc, seq_lens, B, T,
                     causal, block_table, bt_stride_b, max_pages_per_seq, seq_x, bt_x);
  if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;

  const WsLayout wl = ws_layout((int32_t)T, s);
  DecodeParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.q_sb = q_stride_t;
  p.q_st = 0;
  p.q_sh = q_stride_h;
  p.kv = static_cast<const char*>(kv_cache);
  p.num_pages = num_pages;
  p.block_table = bt_x;
  p.bt_sb = max_pages_per_seq;
  p.max_pages = max_pages_per_seq;
  p.seq_lens = seq_x;
  p.B = (int32_t)T;
  p.q_len = 1;
  p.N = N;
  p.n_hg = s.n_hg;
  p.m_wg = s.m_wg;
  p.hg_heads = s.hg_heads;
  p.scale_log2 = softmax_scale * kLog2e;
  p.out = static_cast<uint16_t*>(out);
  p.o_sb = o_stride_t;
  p.o_st = 0;
  p.o_sh = o_stride_h;
  p.lse = lse;
  p.req = reinterpret_cast<int4*>(ws + wl.req);
  p.part_lse = reinterpret_cast<float*>(ws + wl.part_lse);
  p.part_o = reinterpret_cast<float*>(ws + wl.part_o);
  p.num_splits = num_splits;
  p.max_slots = s.max_slots;
  return decode_launch(p, s, kv_dtype, num_splits, (int32_t)T, max_pages_per_seq, di, hs);
}
