/*
 * mla.h -- C ABI of the MI355X (gfx950) MLA paged-latent decode library.
 *
 * Multi-head Latent Attention decode, run as absorbed multi-query attention
 * over a paged cache in which every token stores ONE 576-element row
 * [kv_c (512, RMS-normed latent) | k_pe (64, decoupled-RoPE key)].  Every query
 * head scores against all 576 elements and the 512-element latent doubles as V.
 *
 * Source pages cited below (by title and section):
 *   [vLLM-MLA]   "vLLM 源码完全拆解(三十七):MLA 注意力后端——矩阵吸收之后,576 维
 *                latent KV 如何被四种内核读走"
 *   [TRTLLM-TP]  "TensorRT-LLM 源码完全拆解(十二):注意力层的张量并行"
 *   [Triton-MLA] "Triton und MLA: portable Attention und Latent-Space-Attention"
 *
 * General rules for every call
 * ----------------------------
 * - All tensor pointers are DEVICE pointers owned by the caller; the library
 *   never allocates or frees memory inside a call.  Scratch space for
 *   mla_decode is a caller-provided workspace sized by
 *   mla_decode_workspace_size().
 * - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *   enqueues work on that stream and returns without synchronising, so the
 *   calls can be captured into a HIP graph.  Callers order mla_cache_write
 *   before mla_decode on the same stream (write-before-read, [vLLM-MLA]
 *   §写缓存: the cache update runs before attention in the same step).
 * - bf16 tensors are IEEE bfloat16; all strides are in ELEMENTS of the
 *   tensor's own type.
 * - Host-checkable violations return a status synchronously and enqueue
 *   nothing; nothing falls back silently ([vLLM-MLA] §Cutlass MLA and
 *   [Triton-MLA] §Grenzen und Fehler: unsupported shapes are rejected).
 *   Launch failures return MLA_ERR_HIP.  Device-side preconditions (slot and
 *   page ids in range, unique slots, seq_lens within the block table) are not
 *   checked on the host; an out-of-range id is clamped so that no access
 *   leaves the caller's buffers, and the affected outputs are then undefined.
 * - Only gfx950 is supported; on another device the calls return
 *   MLA_ERR_DEVICE.
 */
#ifndef MLA_PAGED_LATENT_MLA_H
#define MLA_PAGED_LATENT_MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,      /* a required pointer is NULL */
  MLA_ERR_SHAPE = 2,     /* a size is outside the supported range */
  MLA_ERR_DTYPE = 3,     /* unknown kv_dtype */
  MLA_ERR_ALIGN = 4,     /* a pointer or stride is not 16-byte aligned */
  MLA_ERR_WORKSPACE = 5, /* workspace NULL or smaller than required */
  MLA_ERR_HIP = 6,       /* a HIP runtime call or kernel launch failed */
  MLA_ERR_DEVICE = 7     /* the current device is not gfx950 */
} mla_status_t;

/* Cache row formats ([vLLM-MLA] §缓存的形状).
 *   MLA_KV_BF16     : 576 bf16 values, 1152 bytes per row.
 *   MLA_KV_FP8_E4M3 : 576 OCP e4m3fn codes, then float32 k_scale, then float32
 *                     v_scale; 584 bytes per row.  K = code * k_scale (all 576),
 *                     V = code * v_scale (first 512). */
enum { MLA_KV_BF16 = 0, MLA_KV_FP8_E4M3 = 1 };

#define MLA_KV_LORA_RANK 512   /* L  */
#define MLA_ROPE_DIM 64        /* R  */
#define MLA_ROW_ELEMS 576      /* L + R */
#define MLA_QK_NOPE_DIM 128    /* P  */
#define MLA_V_HEAD_DIM 128     /* V  */
#define MLA_PAGE_TOKENS 64     /* tokens per cache page ([vLLM-MLA] §FlashMLA: 64 only) */
#define MLA_MAX_HEADS 128      /* query heads per call ([vLLM-MLA] §Cutlass MLA: MAX_HEADS) */
#define MLA_ROW_BYTES_BF16 1152
#define MLA_ROW_BYTES_FP8 584

/* Upper bound on (request, split) pairs the automatic split planner creates
 * beyond one per request; it bounds the workspace of num_splits == 0. */
#define MLA_AUTO_MAX_EXTRA_PAIRS 1024

/*
 * mla_cache_write -- concat-and-cache scatter ([vLLM-MLA] §写缓存: latent and
 * k_pe of a token are written into one cache row by one kernel, at
 * slot_mapping[t]).
 *
 *   kv_c          bf16 [T, 512], row stride kv_c_stride_t (>= 512, multiple of 8)
 *   k_pe          bf16 [T, 64],  row stride k_pe_stride_t (>= 64, multiple of 8)
 *   slot_mapping  int64 [T] (device): slot = page * 64 + offset; slot < 0 skips
 *                 the token (padding).  Slots must be unique.
 *   kv_cache      pool [num_pages, 64, row] of kv_dtype rows (1152 or 584 bytes)
 *
 * bf16: the row is a bit copy of [kv_c | k_pe].  fp8: per token, amax over the
 * 576 values, s = amax / 448 (IEEE float32 division; s = 1 if amax == 0),
 * code_i = e4m3fn(x_i / s) rounded to nearest-even with saturation to +-448,
 * and s is stored in both scale slots.  Pointers 16-byte aligned.  T may be 0.
 */
mla_status_t mla_cache_write(const void* kv_c, int64_t kv_c_stride_t,
                             const void* k_pe, int64_t k_pe_stride_t,
                             const int64_t* slot_mapping, int64_t T,
                             void* kv_cache, int32_t kv_dtype, int64_t num_pages,
                             void* stream);

/*
 * mla_absorb_q -- query absorption ([vLLM-MLA] §权重准备 and §两套算法:
 * q_l = q_nope . W_UK_T per head with W_UK_T laid out [N, P, L]; [TRTLLM-TP]
 * §吸收: the product is written straight into a [T, N, L + R] fused query whose
 * tail holds q_pe).
 *
 *   q_nope  bf16 [T, N, 128], strides (qn_stride_t, qn_stride_h)
 *   q_pe    bf16 [T, N, 64],  strides (qp_stride_t, qp_stride_h); may be NULL,
 *           then only the first 512 elements of each q_fused row are written
 *   w_uk_t  bf16 [N, 128, 512], contiguous
 *   q_fused bf16 [T, N, 576], strides (qf_stride_t, qf_stride_h)
 *
 * q_fused[t,h,0:512] = bf16_rne(sum_p q_nope[t,h,p] * W_UK_T[h,p,:]) with
 * float32 accumulation; q_fused[t,h,512:576] = q_pe[t,h,:].
 * 1 <= N <= 128, T >= 0.  Pointers 16-byte aligned, strides multiples of 8.
 */
mla_status_t mla_absorb_q(const void* q_nope, int64_t qn_stride_t, int64_t qn_stride_h,
                          const void* q_pe, int64_t qp_stride_t, int64_t qp_stride_h,
                          const void* w_uk_t, int64_t T, int32_t N,
                          void* q_fused, int64_t qf_stride_t, int64_t qf_stride_h,
                          void* stream);

/*
 * mla_absorb_q_cache_write -- mla_absorb_q and mla_cache_write in one launch (the
 * two steps the pages place before attention in a decode step, [vLLM-MLA] §写缓存
 * and §两套算法): the cache rows of the step's T_new new tokens are written by
 * workgroups launched beside the absorption's, so the step pays one launch for
 * both.  The two operations are independent (the absorption reads no cache row).
 *
 *   q_nope .. qf_stride_h     as mla_absorb_q (T query rows, N heads)
 *   kv_c .. num_pages         as mla_cache_write (T_new rows into kv_cache)
 *
 * Results are bit for bit those of the two calls; statuses are theirs (checked
 * before anything is enqueued); additionally MLA_ERR_SHAPE when N plus
 * ceil(T_new / 16) exceeds 65535 grid rows.  T == 0 runs the cache write alone.
 */
mla_status_t mla_absorb_q_cache_write(const void* q_nope, int64_t qn_stride_t, int64_t qn_stride_h,
                                      const void* q_pe, int64_t qp_stride_t, int64_t qp_stride_h,
                                      const void* w_uk_t, int64_t T, int32_t N,
                                      void* q_fused, int64_t qf_stride_t, int64_t qf_stride_h,
                                      const void* kv_c, int64_t kv_c_stride_t,
                                      const void* k_pe, int64_t k_pe_stride_t,
                                      const int64_t* slot_mapping, int64_t T_new,
                                      void* kv_cache, int32_t kv_dtype, int64_t num_pages,
                                      void* stream);

/*
 * mla_absorb_q_rope -- mla_absorb_q with the rotary position embedding of q_pe
 * applied on the way into the tail ([vLLM-MLA] §从模型层看: the model layer
 * rotates the last 64 query values by rotary_emb(positions, ...) before MLA;
 * [TRTLLM-TP] §吸收: the rotation runs beside the absorption GEMM).
 *
 *   q_nope, w_uk_t, q_fused  as mla_absorb_q; q_pe is required
 *   positions      int64 [T] (device): the token's position
 *   cos_sin_cache  float32 [max_pos, 64] contiguous, 16-byte aligned:
 *                  row p = [cos(p w_0) .. cos(p w_31) | sin(p w_0) .. sin(p w_31)]
 *   neox           nonzero: rotate-half pairing (value i with i + 32, frequency i);
 *                  zero: adjacent pairs (value 2i with 2i + 1, frequency i)
 *
 * Pair (a, b) of frequency i -> (a cos - b sin, b cos + a sin), float32, bf16
 * RNE.  A token whose position is outside [0, max_pos) gets a NaN tail (64
 * quiet NaNs), so a bad position shows in the scores rather than passing
 * silently.  The frequency schedule (base, scaling) is the table's business.
 */
mla_status_t mla_absorb_q_rope(const void* q_nope, int64_t qn_stride_t, int64_t qn_stride_h,
                               const void* q_pe, int64_t qp_stride_t, int64_t qp_stride_h,
                               const void* w_uk_t, int64_t T, int32_t N, const int64_t* positions,
                               const float* cos_sin_cache, int64_t max_pos, int32_t neox,
                               void* q_fused, int64_t qf_stride_t, int64_t qf_stride_h,
                               void* stream);

/*
 * mla_decode_workspace_size -- bytes of workspace mla_decode needs for this
 * batch shape and split mode (see num_splits below).  Returns 0 for shapes
 * mla_decode would reject.  Pure host arithmetic; no device call.
 */
size_t mla_decode_workspace_size(int32_t B, int32_t q_len, int32_t N, int32_t num_splits);

/*
 * mla_decode -- paged split-KV absorbed-MQA decode with an LSE split merge
 * ([vLLM-MLA] §两套算法 data-movement-friendly form, §FlashMLA, §Triton MLA;
 * [Triton-MLA] §Datenfluss).
 *
 *   q            bf16 [B, q_len, N, 576] absorbed query, strides
 *                (q_stride_b, q_stride_t, q_stride_h); last dim contiguous
 *   kv_cache     pool [num_pages, 64, row] (kv_dtype rows)
 *   block_table  int32 [B, max_pages_per_seq], row stride bt_stride_b: logical
 *                page j of request b is physical page block_table[b][j];
 *                entries past ceil(seq_lens[b] / 64) are never read (nor
 *                past 2^25 - 1 pages: no int32 seq_len reaches further)
 *   seq_lens     int32 [B] (device): cached tokens of request b INCLUDING the
 *                q_len new ones; query row t sees tokens
 *                [0, seq_lens[b] - q_len + 1 + t) (causal within the q_len
 *                block, [vLLM-MLA] §Triton MLA); a row that sees no token gets
 *                o = 0 and lse = -inf
 *   softmax_scale  applied to q.k (pass 1/sqrt(192) for DeepSeek-V3: the scale
 *                keeps the un-absorbed 192-wide value, [vLLM-MLA] §两套算法)
 *   num_splits   0 = automatic plan from seq_lens and the device's compute
 *                units; 1 = one split per request (batch-invariant reduction
 *                order, [vLLM-MLA] §FlashMLA batch-invariance); k > 1 = each
 *                request split into up to k page-aligned pieces (k <= 4096)
 *   workspace    device scratch of at least mla_decode_workspace_size() bytes,
 *                256-byte aligned; its contents need no initialisation.  It
 *                holds the split table and the split partials (per partial row
 *                a float32 LSE and 512 float32 values)
 *   out          bf16 [B, q_len, N, 512], strides (o_stride_b, o_stride_t,
 *                o_stride_h); last dim contiguous
 *   lse          float32 [B, q_len, N] contiguous: natural-log log-sum-exp of
 *                the scaled scores ([Triton-MLA] §Entwurfsmotivation)
 *
 * Limits: 1 <= B, q_len in {1, 2}, 1 <= N <= 128.  q, out, kv_cache and
 * workspace 16-byte aligned (workspace 256), strides multiples of 8.  The
 * result is deterministic for fixed inputs and num_splits; across different
 * batch compositions only num_splits == 1 keeps bit-identical per-request
 * results.  No host synchronisation, no allocation.
 */
mla_status_t mla_decode(const void* q, int64_t q_stride_b, int64_t q_stride_t, int64_t q_stride_h,
                        const void* kv_cache, int32_t kv_dtype, int64_t num_pages,
                        const int32_t* block_table, int64_t bt_stride_b, int32_t max_pages_per_seq,
                        const int32_t* seq_lens, int32_t B, int32_t q_len, int32_t N,
                        float softmax_scale, int32_t num_splits,
                        void* workspace, size_t workspace_bytes,
                        void* out, int64_t o_stride_b, int64_t o_stride_t, int64_t o_stride_h,
                        float* lse, void* stream);

/*
 * mla_decode_noalloc -- mla_decode for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, runtimes that forbid
 * hipMalloc): the same kernels, split plan and merge, with the split table and
 * partials in a scratch array the library keeps on every GPU it runs on
 * (MLA_DECODE_SCRATCH_BYTES, a file-scope device array held until the process ends)
 * instead of a caller workspace.
 *
 *   arguments  as mla_decode, without workspace / workspace_bytes
 *
 * The scratch needs (B + S + 8) * groups * rows * 2052 bytes plus a 16-byte record
 * per request, where S is the automatic plan's stream count on this GPU (its compute
 * units, divided among head groups) or B * num_splits, groups * rows = q_len * N
 * rounded up to 16 (q_len * N <= 16) or 64; num_splits == 1 needs only the records.
 * Shapes that need more than MLA_DECODE_SCRATCH_BYTES return MLA_ERR_WORKSPACE and
 * enqueue nothing (the 128-head benchmark batches of up to 128 requests fit).  The
 * call allocates and frees nothing; the scratch needs no initialisation and keeps the
 * last call's contents.  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (concurrent streams, or host threads enqueuing on different
 * streams) race and give undefined results; calls ordered on one stream are safe.
 * Same results as mla_decode for the same inputs and num_splits.
 */
#define MLA_DECODE_SCRATCH_BYTES (96u << 20)
mla_status_t mla_decode_noalloc(const void* q, int64_t q_stride_b, int64_t q_stride_t, int64_t q_stride_h,
                                const void* kv_cache, int32_t kv_dtype, int64_t num_pages,
                                const int32_t* block_table, int64_t bt_stride_b, int32_t max_pages_per_seq,
                                const int32_t* seq_lens, int32_t B, int32_t q_len, int32_t N,
                                float softmax_scale, int32_t num_splits,
                                void* out, int64_t o_stride_b, int64_t o_stride_t, int64_t o_stride_h,
                                float* lse, void* stream);

/*
 * mla_decode_varlen_workspace_size -- bytes of workspace mla_decode_varlen needs
 * for T query rows of N heads, the split mode and the block-table width.
 * Returns 0 for shapes mla_decode_varlen would reject.  No device call.
 */
size_t mla_decode_varlen_workspace_size(int64_t T, int32_t N, int32_t num_splits,
                                        int32_t max_pages_per_seq);

/*
 * mla_decode_varlen -- decode with a different number of query tokens per
 * request ([vLLM-MLA] §投机解码 and §Metadata, QueryLenSupport VARLEN: a
 * verification batch mixes 1-, 2-, 3-token queries; causal blocks give each row
 * its own sequence length, non-causal draft blocks give every row the whole
 * prefix).
 *
 *   q                bf16 [T, N, 576] flat query rows, strides (q_stride_t,
 *                    q_stride_h); request b owns rows query_start_loc[b] ..
 *                    query_start_loc[b + 1] - 1
 *   query_start_loc  int32 [B + 1] (device), non-decreasing, [0] = 0, [B] = T
 *   seq_lens         int32 [B] (device): cached tokens of request b including
 *                    its query_len new ones
 *   causal           nonzero: row t of a q-token block sees seq_lens[b] - q + 1 + t
 *                    tokens; zero: every row sees seq_lens[b] tokens
 *   out              bf16 [T, N, 512], strides (o_stride_t, o_stride_h)
 *   lse              float32 [T, N] contiguous
 *   other arguments  as mla_decode; workspace of mla_decode_varlen_workspace_size()
 *                    bytes (it holds each row's length and a copy of its request's
 *                    block-table row, T * max_pages_per_seq int32)
 *
 * Each row runs as a one-row decode (same kernels, same split plan and merge),
 * so a request's pages are read once per query row.  Rows outside every
 * request's range see no token (o = 0, lse = -inf).  T <= 2^24.
 */
mla_status_t mla_decode_varlen(const void* q, int64_t q_stride_t, int64_t q_stride_h,
                               const void* kv_cache, int32_t kv_dtype, int64_t num_pages,
                               const int32_t* block_table, int64_t bt_stride_b,
                               int32_t max_pages_per_seq, const int32_t* query_start_loc,
                               const int32_t* seq_lens, int32_t B, int64_t T, int32_t N,
                               int32_t causal, float softmax_scale, int32_t num_splits,
                               void* workspace, size_t workspace_bytes, void* out,
                               int64_t o_stride_t, int64_t o_stride_h, float* lse, void* stream);

/*
 * mla_up_v -- per-head V up-projection of the latent attention output
 * ([vLLM-MLA] §两套算法, _v_up_proj: [N, T, L] @ W_UV[N, L, V] written through a
 * transposed view into a token-major [T, N * V] buffer).
 *
 *   o_lat  bf16 [T, N, 512], strides (ol_stride_t, ol_stride_h)
 *   w_uv   bf16 [N, 512, 128], contiguous
 *   out    bf16 [T, N * 128]: head h of token t at out + t*out_stride_t + h*128
 *
 * out[t, h*128 + v] = bf16_rne(sum_l o_lat[t,h,l] * W_UV[h,l,v]), float32
 * accumulation.  1 <= N <= 128, T >= 0.  16-byte alignment as above.
 */
mla_status_t mla_up_v(const void* o_lat, int64_t ol_stride_t, int64_t ol_stride_h,
                      const void* w_uv, int64_t T, int32_t N,
                      void* out, int64_t out_stride_t, void* stream);

/*
 * mla_up_v_fp8 -- mla_up_v with its output quantized to fp8 per token group
 * ([vLLM-MLA] §QuantKey: when the next layer takes fp8 input, the W_UV output is
 * quantized dynamically in groups of 128 or 64 consecutive elements of a token,
 * one float32 scale per group).
 *
 *   o_lat, w_uv  as mla_up_v
 *   group        64 or 128
 *   out_codes    uint8 [T, N * 128] e4m3fn codes, row stride codes_stride_t bytes
 *                (>= N * 128, multiple of 8; 8-byte aligned)
 *   out_scales   float32 [T, N * 128 / group], row stride scales_stride_t
 *                elements (>= N * 128 / group; 4-byte aligned)
 *
 * y = the bf16 value mla_up_v writes; for each group g of a token
 * s = fl32(amax_g |y| / 448) (s = 1 for an all-zero group), code = e4m3fn of
 * fl32(y / s), round to nearest even, saturating at +-448.  The scale rule is the
 * one the fp8 cache rows use; the page names the grouping only.  Results are
 * defined for finite y.  1 <= N <= 128, 0 <= T <= 65535 * 32.
 */
mla_status_t mla_up_v_fp8(const void* o_lat, int64_t ol_stride_t, int64_t ol_stride_h,
                          const void* w_uv, int64_t T, int32_t N, int32_t group,
                          void* out_codes, int64_t codes_stride_t, float* out_scales,
                          int64_t scales_stride_t, void* stream);

/*
 * mla_kv_b_proj -- up-projection of latents into prefill keys and values
 * ([vLLM-MLA] §Prefill: kv_b_proj(kv_c) gives k_nope and v of the new tokens;
 * §两套算法, compute-friendly form).
 *
 *   kv_c   bf16 [S, 512], row stride kc_stride_t (the latent part of cache rows)
 *   w_kvb  bf16 [N, 512, 256] contiguous: per head [W_UK[h] | W_UV[h]] (P = 128
 *          key columns, then V = 128 value columns)
 *   out    bf16 [S, N, 256], strides (out_stride_t, out_stride_h):
 *          k_nope = out[..., 0:128], v = out[..., 128:256]
 *
 * out[s,h,:] = bf16_rne(sum_l kv_c[s,l] * w_kvb[h,l,:]), float32 accumulation.
 * 1 <= N <= 128, S >= 0.  16-byte alignment, strides multiples of 8.
 */
mla_status_t mla_kv_b_proj(const void* kv_c, int64_t kc_stride_t, const void* w_kvb, int64_t S,
                           int32_t N, void* out, int64_t out_stride_t, int64_t out_stride_h,
                           void* stream);

/*
 * mla_prefill_mha -- attention of the new tokens of a prefill batch
 * ([vLLM-MLA] §Prefill, run_prefill_new_tokens: keys [k_nope | k_pe] with the one
 * rope key broadcast over heads (192 wide), values 128 wide, softmax scale
 * 1/sqrt(192); the output and LSE merge with a context part through
 * mla_merge_attn_states).
 *
 *   q             bf16 [T, N, 192] ([q_nope | q_pe]), strides (q_stride_t, q_stride_h)
 *   k_nope        bf16 [S, N, 128], strides (kn_stride_t, kn_stride_h)
 *   k_pe          bf16 [S, 64], row stride kp_stride_t
 *   v             bf16 [S, N, 128], strides (v_stride_t, v_stride_h)
 *   cu_seqlens_q  int32 [B + 1] (device): request b owns query rows [cu_q[b], cu_q[b+1])
 *   cu_seqlens_k  int32 [B + 1] (device): and keys [cu_k[b], cu_k[b+1])
 *   max_q_len     the longest request's query rows (rows past it are not written)
 *   causal        nonzero: query row i of a request with qlen rows and klen keys
 *                 sees keys 0 .. klen - qlen + i; zero: all klen keys
 *   out           bf16 [T, N, 128], strides (o_stride_t, o_stride_h)
 *   lse           float32 [T, N] contiguous, natural log of the scaled scores
 *
 * A row that sees no key gets o = 0, lse = -inf.  Request bounds are clamped to
 * [0, T] and [0, S].  1 <= N <= 128, 0 <= B <= 65535, T, S < 2^31.  Pointers
 * 16-byte aligned (lse and cu arrays 4), strides multiples of 8.
 */
mla_status_t mla_prefill_mha(const void* q, int64_t q_stride_t, int64_t q_stride_h, const void* k_nope,
                             int64_t kn_stride_t, int64_t kn_stride_h, const void* k_pe,
                             int64_t kp_stride_t, const void* v, int64_t v_stride_t, int64_t v_stride_h,
                             const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t B,
                             int64_t T, int64_t S, int32_t N, int32_t max_q_len, int32_t causal,
                             float softmax_scale, void* out, int64_t o_stride_t, int64_t o_stride_h,
                             float* lse, void* stream);

/*
 * mla_prefill_workspace_rows -- the row budget W of the chunked-context workspace
 * ([vLLM-MLA] §Prefill, the workspace-size formula):
 * W = min(max(8 * max_model_len, 4 * max_num_seqs * page_tokens), 64 * 1024).
 * Host arithmetic; 0 for a non-positive argument.
 */
int64_t mla_prefill_workspace_rows(int64_t max_model_len, int64_t max_num_seqs, int32_t page_tokens);

/*
 * mla_plan_context_chunks -- chunk plan of a prefill batch's context ([vLLM-MLA]
 * §Prefill: the requests' context rows are packed in request order into chunks of at
 * most row_budget rows; a request that does not fit in what is left of a chunk is cut
 * on a 64-token page boundary and continues in the next chunk, so every chunk starts a
 * request on a page boundary, as mla_gather_cache requires).  Host arithmetic on host
 * arrays; no device call.
 *
 *   context_lens  int32 [B] (host): context tokens of each request (<= 0: none)
 *   row_budget    rows per chunk, 64 <= row_budget < 2^31 (e.g. mla_prefill_workspace_rows)
 *   chunk_starts  int32 [max_chunks, B] (host) or NULL: first context token of request
 *                 b in chunk c (a multiple of 64), 0 where b has no rows in c
 *   chunk_lens    int32 [max_chunks, B] (host) or NULL: its tokens in chunk c (0: none)
 *
 * Returns the number of chunks (call with max_chunks = 0 to size the arrays); only
 * the first max_chunks are written.  Negative: -MLA_ERR_NULL or -MLA_ERR_SHAPE.  Per
 * chunk, cu_seq_lens is the prefix sum of its lens and seq_starts its starts (for
 * mla_gather_cache), and the same prefix sum is the chunk's cu_seqlens_k for
 * mla_prefill_mha of the new tokens (not causal).  fp8 caches: the gather upconverts a
 * row with its K scale, so the prefill path takes V from code * k_scale; rows written
 * by mla_cache_write carry equal K and V scales.
 */
int64_t mla_plan_context_chunks(const int32_t* context_lens, int32_t B, int64_t row_budget,
                                int32_t* chunk_starts, int32_t* chunk_lens, int64_t max_chunks);

/*
 * mla_gather_cache -- gather context rows of the paged cache into a contiguous
 * bf16 workspace ([vLLM-MLA] §Prefill, chunked context: the rows a chunk needs
 * are collected by block_table, cu_seq_lens and token_to_seq so that kv_b_proj
 * runs as one GEMM; fp8 rows are upconverted to bf16 while gathering; a chunk
 * starts on a page boundary of its request).
 *
 *   kv_cache      pool [num_pages, 64, row] (kv_dtype rows), read only
 *   block_table   int32 [B, max_pages_per_seq], row stride bt_stride_b
 *   cu_seq_lens   int32 [B + 1] (device): rows of request b go to output rows
 *                 [cu_seq_lens[b], cu_seq_lens[b + 1])
 *   seq_starts    int32 [B] (device) or NULL (all 0): the request's first token
 *                 in this chunk
 *   token_to_seq  int32 [total_rows] (device): the request of each output row
 *   out           bf16 [total_rows, 576], row stride out_stride (elements)
 *
 * Output row r of request b = token_to_seq[r] is logical token
 * j = seq_starts[b] + r - cu_seq_lens[b] of b, at page block_table[b][j / 64],
 * offset j % 64.  bf16 rows are copied bit for bit; an fp8 row becomes
 * bf16_rne(code * k_scale) for all 576 elements (its K view; rounded once from
 * the exact product).  A row whose request, token or page id is out of range
 * is written as zeros.  Only the output is written.  kv_cache and out 16-byte
 * aligned, out_stride a multiple of 8.
 */
mla_status_t mla_gather_cache(const void* kv_cache, int32_t kv_dtype, int64_t num_pages,
                              const int32_t* block_table, int64_t bt_stride_b,
                              int32_t max_pages_per_seq, const int32_t* cu_seq_lens,
                              const int32_t* seq_starts, const int32_t* token_to_seq, int32_t B,
                              int64_t total_rows, void* out, int64_t out_stride, void* stream);

/*
 * mla_merge_attn_states -- merge two attention states of the same query rows
 * over disjoint key sets ([vLLM-MLA] §Prefill, merge_attn_states: the context
 * result and the new-token result are re-weighted by exp(lse - max_lse) per
 * head and row; a state with no keys, o = 0 and lse = -inf, weighs zero).
 *
 *   prefix_out, suffix_out, out   bf16 [T, N, D], element strides
 *                                 (o_stride_t, o_stride_h), last dim contiguous
 *   prefix_lse, suffix_lse, out_lse  float32 [T, N], element strides
 *                                 (lse_stride_t, lse_stride_h); out_lse may be NULL
 *
 * With w_x = exp(lse_x - m), m = max(lse_p, lse_s):
 * out = bf16_rne((w_p o_p + w_s o_s) / (w_p + w_s)), out_lse = m + ln(w_p + w_s)
 * (float32); both states empty gives out = 0, out_lse = -inf.  1 <= N,
 * 8 <= D <= 4096 with D a multiple of 8; tensors 16-byte aligned, o strides
 * multiples of 8.  out may alias neither input.
 */
mla_status_t mla_merge_attn_states(const void* prefix_out, const float* prefix_lse,
                                   const void* suffix_out, const float* suffix_lse, int64_t T,
                                   int32_t N, int32_t D, int64_t o_stride_t, int64_t o_stride_h,
                                   int64_t lse_stride_t, int64_t lse_stride_h, void* out,
                                   float* out_lse, void* stream);

/* Human-readable name of a status code (static string). */
const char* mla_status_str(mla_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PAGED_LATENT_MLA_H */
