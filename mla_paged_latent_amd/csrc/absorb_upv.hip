// Per-head batched contractions around the decode kernel:
//   mla_absorb_q : q_fused[t,h,0:512] = q_nope[t,h,:] . W_UK_T[h]   (K = 128, N = 512)
//                  q_fused[t,h,512:576] = q_pe[t,h,:]
//   mla_up_v     : out[t, h*128 : h*128+128] = o_lat[t,h,:] . W_UV[h] (K = 512, N = 128)
// Source: "vLLM 源码完全拆解(三十七):MLA 注意力后端", §权重准备 (W_UK_T is [N, P, L],
// W_UV is [N, L, V], one batched GEMM over heads) and §两套算法 (absorption into the
// query; _v_up_proj writing token-major through a transposed view); "TensorRT-LLM
// 源码完全拆解(十二)", §吸收 (the absorbed query is written into the front of a
// [T, N, L + R] buffer whose tail holds q_pe).
//
// Both weights are stored [K][N] with N contiguous while the MFMA wants K contiguous
// per lane, so a workgroup stages its head's [K x NT] weight tile in LDS and reads it
// with ds_read_b64_tr_b16 (a 4-row x 16-column transpose per 16 lanes).  The product
// is formed transposed, D^T[n][t] = W^T[n][k] . A^T[k][t], on 32x32x16 bf16 MFMAs:
// W^T is the A operand (rows n), activation rows come straight from HBM as the B
// operand (16 contiguous bytes of one token row per lane), and each lane of the
// accumulator holds 4 consecutive n of one token; the 32-token tile is staged in LDS
// and leaves as contiguous row segments.
#include "cache_rows.h"
#include "mla_common.h"
#include "mla_host.h"

namespace mla {

template <int KK, int NN, int NT, int KSPLIT>
struct GemmCfg {
  static constexpr int kNB = NT / 32;                 // 32-wide n blocks per tile
  static_assert(kNB * KSPLIT == 4, "4 waves per workgroup");
  static constexpr int kKPerWave = KK / KSPLIT;
  static constexpr int kKSteps = kKPerWave / 16;
  static constexpr int kRowBytes = NT * 2 + 32;       // padded LDS row: 4 rows hit disjoint banks
  static constexpr int kTileBytes = KK * kRowBytes;
  static constexpr int kRedBytes = (KSPLIT > 1) ? (kNB * 32 * 32 * 4) : 0;
  static constexpr int kOutPitch = NT * 2 + 16;       // output staging row (32 tokens x NT)
  static constexpr int kOutBytes = 32 * kOutPitch;
  static constexpr int kAPitch = KK * 2 + 16;         // activation staging row (32 tokens x KK)
  static constexpr int kABytes = 32 * kAPitch;
  static constexpr int kAPerThread = 32 * KK / 8 / 256;   // 16-byte chunks per thread
  static constexpr int kLdsBytes = kTileBytes + kRedBytes + kOutBytes + kABytes;
};

// What head_gemm_kernel writes after the NN product columns of each row.
enum PeTail { kNoTail = 0, kCopyTail = 1, kRopeTail = 2 };

// Rotary position embedding of one token's 16 rope values that share the
// frequencies f0 .. f0+7 (f0 = 8 * c): with rotate-half pairing they are
// chunks c and c + 4 of the 64-value row (value i pairs with i + 32), with
// adjacent pairing chunks 2c and 2c + 1 (value 2k pairs with 2k + 1, frequency
// k).  Pair (a, b) -> (a cos - b sin, b cos + a sin) in float32, bf16 RNE.
// cs = cos(f0..f0+7), sin(f0..f0+7).  A position outside the table gives NaN.
__device__ __forceinline__ void rope_chunks(const uint4& xa, const uint4& xb, const float (&cs)[16],
                                            bool ok, bool neox, uint4& ya, uint4& yb) {
  const uint32_t in[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
  float v[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[2 * i] = bf16_bits_to_f32(in[i] & 0xFFFFu);
    v[2 * i + 1] = bf16_bits_to_f32(in[i] >> 16);
  }
  float r[16];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    // the pair of frequency f0 + j: (v[ia], v[ib])
    const int ia = neox ? j : 2 * j, ib = neox ? j + 8 : 2 * j + 1;
    r[ia] = v[ia] * cs[j] - v[ib] * cs[8 + j];
    r[ib] = v[ib] * cs[j] + v[ia] * cs[8 + j];
  }
  uint32_t out[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bf16x2_t pr = {(__bf16)r[2 * i], (__bf16)r[2 * i + 1]};
    out[i] = ok ? __builtin_bit_cast(uint32_t, pr) : 0x7FC07FC0u;
  }
  ya = uint4{out[0], out[1], out[2], out[3]};
  yb = uint4{out[4], out[5], out[6], out[7]};
}

// Cache rows written beside the absorption in the same launch (mla_absorb_q_cache_write):
// the first grid rows' workgroups write four tokens each and the heads follow, so the
// row writes are dispatched first and end inside the absorption's time.
struct CacheRowsArgs {
  const uint16_t* kv_c;
  int64_t kv_stride;
  const uint16_t* k_pe;
  int64_t pe_stride;
  const int64_t* slots;
  int64_t T;
  char* pool;
  int64_t num_pages;
  int32_t row_lines;   // grid rows [0, row_lines) write cache rows, the heads follow
};
constexpr int kNoRows = 0, kRowsBf16 = 1, kRowsFp8 = 2;

// grid = (NN / NT, N heads [+ cache-row workgroups, CW]); block = 256 threads.
template <int KK, int NN, int NT, int KSPLIT, int PE, int CW = kNoRows>
__global__ __launch_bounds__(256) void head_gemm_kernel(
    const uint16_t* __restrict__ A, int64_t a_st, int64_t a_sh,      // [T, N, KK]
    const uint16_t* __restrict__ W,                                   // [N, KK, NN]
    uint16_t* __restrict__ C, int64_t c_st, int64_t c_sh,            // [T, N, NN]
    const uint16_t* __restrict__ pe, int64_t pe_st, int64_t pe_sh,   // [T, N, 64] (PE != 0)
    const int64_t* __restrict__ positions,                            // [T] (kRopeTail)
    const float* __restrict__ cos_sin, int64_t max_pos, int neox,     // [max_pos, 64] (kRopeTail)
    int64_t T, CacheRowsArgs cw) {
  using Cfg = GemmCfg<KK, NN, NT, KSPLIT>;
  __shared__ __attribute__((aligned(16))) char smem[Cfg::kLdsBytes];
  MLA_LDS char* lds = (MLA_LDS char*)(smem);
  if constexpr (CW != kNoRows) {
    if ((int)blockIdx.y < cw.row_lines) {
      const int64_t t = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * 4 + (threadIdx.x >> 6);
      if (t < cw.T)
        cache_write_row<CW == kRowsFp8>(cw.kv_c, cw.kv_stride, cw.k_pe, cw.pe_stride, cw.slots, cw.pool,
                                        cw.num_pages, t, lane_id());
      return;
    }
  }

  const int h = (int)blockIdx.y - (CW != kNoRows ? cw.row_lines : 0);
  const int n0 = blockIdx.x * NT;
  const int tid = threadIdx.x;
  const int w = wave_id();
  const int l = lane_id();

  // The first tokens' q_pe chunks (n-tile 0), W[h][0:KK][n0:n0+NT] and the first token
  // block's activation fragments are all requested before anything waits, so a
  // workgroup keeps its whole tile in flight.  A copied tail moves one 16-byte chunk
  // per item (8 per token); a rotated tail two chunks that share 8 frequencies (4 per
  // token), chunks c and c + 4 (rotate-half) or 2c and 2c + 1 (adjacent pairs).
  const bool do_pe = PE != kNoTail && blockIdx.x == 0;
  constexpr int kPeItems = PE == kRopeTail ? 4 : 8;
  auto pe_chunks = [&](int c, int& ca, int& cb) {
    ca = PE == kRopeTail ? (neox ? c : 2 * c) : c;
    cb = neox ? c + 4 : 2 * c + 1;
  };
  uint4 pe_v, pe_w;
  int64_t pos_v = 0;
  const bool pe_first = do_pe && tid < T * kPeItems;
  if (pe_first) {
    const int t = tid / kPeItems, c = tid % kPeItems;
    int ca, cb;
    pe_chunks(c, ca, cb);
    if (PE == kRopeTail) pos_v = positions[t];
    pe_v = *reinterpret_cast<const uint4*>(pe + t * pe_st + h * pe_sh + ca * 8);
    if (PE == kRopeTail) pe_w = *reinterpret_cast<const uint4*>(pe + t * pe_st + h * pe_sh + cb * 8);
  }
  const uint16_t* wh = W + (int64_t)h * KK * NN + n0;
  constexpr int kChunksPerRow = NT / 8;
  constexpr int kTileChunks = KK * kChunksPerRow;
  static_assert(kTileChunks % 256 == 0, "tile chunks per thread");
  constexpr int kPerThread = kTileChunks / 256;
  // no other workgroup reads this W tile: nontemporal loads (the full_head decode step,
  // whose KV stream leaves the weights cold, measured 110.1 -> 108.4 us with them)
  u32x4_t wv[kPerThread];
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int i = tid + 256 * j;
    const int k = i / kChunksPerRow, c = i % kChunksPerRow;
    wv[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(wh + (int64_t)k * NN + c * 8));
  }
  // the rotation's table row, once the position has arrived
  auto load_cs = [&](int64_t pos, int c, float (&cs)[16]) -> bool {
    const bool ok = pos >= 0 && pos < max_pos;
    const float* row = cos_sin + (ok ? pos : 0) * 64 + 8 * c;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const float4 a = *reinterpret_cast<const float4*>(row + 4 * q);
      const float4 b = *reinterpret_cast<const float4*>(row + 32 + 4 * q);
      cs[4 * q] = a.x; cs[4 * q + 1] = a.y; cs[4 * q + 2] = a.z; cs[4 * q + 3] = a.w;
      cs[8 + 4 * q] = b.x; cs[8 + 4 * q + 1] = b.y; cs[8 + 4 * q + 2] = b.z; cs[8 + 4 * q + 3] = b.w;
    }
    return ok;
  };
  float cs_v[16];
  bool pos_ok = false;
  if (PE == kRopeTail && pe_first) pos_ok = load_cs(pos_v, tid % kPeItems, cs_v);

  const int nb = w % Cfg::kNB;          // n block of this wave
  const int kh = w / Cfg::kNB;          // K slice of this wave
  const int g = l >> 4, lg = l & 15;
  // transpose-read address pieces: 16-lane group g covers n = 16*(g&1) + [0,16) and
  // k rows 8*(g>>1) + 4*r + (lg>>2) for read r; lane supplies column 4*(lg&3).
  const uint32_t tr_col = (uint32_t)((nb * 32 + 16 * (g & 1) + 4 * (lg & 3)) * 2);
  const int tr_row0 = 8 * (g >> 1) + (lg >> 2);

  // A token block's activations are staged in LDS: consecutive lanes read consecutive
  // 16-byte chunks of a token row (whole cache lines per instruction), and each lane
  // then takes its MFMA fragment (one token, 8 consecutive k) from LDS.  Read straight
  // from HBM in fragment order, every instruction would touch 32 rows for 32 bytes
  // each, and the activation reads would cost twice what the rest of the kernel does.
  // The next block's chunks are loaded while the current block is multiplied.
  MLA_LDS char* astage = lds + Cfg::kTileBytes + Cfg::kRedBytes + Cfg::kOutBytes;
  constexpr int kRowChunksA = KK / 8;
  u32x4_t av[Cfg::kAPerThread];
  auto load_act = [&](int64_t tb) {
#pragma unroll
    for (int j = 0; j < Cfg::kAPerThread; ++j) {
      const int i = tid + 256 * j;
      const int64_t t = tb + i / kRowChunksA;
      av[j] = t < T ? *reinterpret_cast<const u32x4_t*>(A + t * a_st + h * a_sh + (i % kRowChunksA) * 8)
                    : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  auto stage_act = [&]() {
#pragma unroll
    for (int j = 0; j < Cfg::kAPerThread; ++j) {
      const int i = tid + 256 * j;
      *reinterpret_cast<MLA_LDS u32x4_t*>(astage + (i / kRowChunksA) * Cfg::kAPitch + (i % kRowChunksA) * 16) =
          av[j];
    }
  };
  load_act(0);

#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int i = tid + 256 * j;
    const int k = i / kChunksPerRow, c = i % kChunksPerRow;
    *reinterpret_cast<MLA_LDS u32x4_t*>(lds + k * Cfg::kRowBytes + c * 16) = wv[j];
  }
  stage_act();
  auto put_tail = [&](int64_t t, int c, const uint4& a, const uint4& b, const float (&cs)[16], bool ok) {
    int ca, cb;
    pe_chunks(c, ca, cb);
    uint16_t* dst = C + t * c_st + h * c_sh + NN;
    if (PE == kCopyTail) {
      *reinterpret_cast<uint4*>(dst + ca * 8) = a;
    } else {
      uint4 ya, yb;
      rope_chunks(a, b, cs, ok, neox != 0, ya, yb);
      *reinterpret_cast<uint4*>(dst + ca * 8) = ya;
      *reinterpret_cast<uint4*>(dst + cb * 8) = yb;
    }
  };
  if (pe_first) put_tail(tid / kPeItems, tid % kPeItems, pe_v, pe_w, cs_v, pos_ok);
  if (do_pe) {
    for (int64_t i = tid + 256; i < T * kPeItems; i += 256) {
      const int64_t t = i / kPeItems;
      const int c = (int)(i % kPeItems);
      int ca, cb;
      pe_chunks(c, ca, cb);
      uint4 a = *reinterpret_cast<const uint4*>(pe + t * pe_st + h * pe_sh + ca * 8), b = a;
      float cs[16];
      bool ok = false;
      if (PE == kRopeTail) {
        b = *reinterpret_cast<const uint4*>(pe + t * pe_st + h * pe_sh + cb * 8);
        ok = load_cs(positions[t], c, cs);
      }
      put_tail(t, c, a, b, cs, ok);
    }
  }
  lds_barrier();

  for (int64_t tb = 0; tb < T; tb += 32) {
    const bool more = tb + 32 < T;
    if (more) load_act(tb + 32);
    f32x16_t acc = {};
#pragma unroll
    for (int ks = 0; ks < Cfg::kKSteps; ++ks) {
      const int k0 = kh * Cfg::kKPerWave + ks * 16;
      const uint32_t r0 = (uint32_t)((k0 + tr_row0) * Cfg::kRowBytes) + tr_col;
      const bf16x4_t lo = lds_read_tr16(lds, r0);
      const bf16x4_t hi = lds_read_tr16(lds, r0 + 4 * Cfg::kRowBytes);
      const bf16x8_t a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const bf16x8_t b = *reinterpret_cast<const MLA_LDS bf16x8_t*>(astage + (l & 31) * Cfg::kAPitch +
                                                                     (k0 + 8 * (l >> 5)) * 2);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
    }
    if constexpr (KSPLIT > 1) {
      // waves with kh > 0 hand their partial tile to the kh == 0 wave of the same n block
      MLA_LDS float* red = reinterpret_cast<MLA_LDS float*>(lds + Cfg::kTileBytes);
      if (kh == 1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) red[(nb * 16 + i) * 64 + l] = acc[i];
      }
      lds_barrier();
      if (kh == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] += red[(nb * 16 + i) * 64 + l];
      }
      lds_barrier();
    }
    // The tile goes out through LDS so that every token's NT outputs leave as whole
    // contiguous row segments (16 B per lane) rather than as 8-byte pieces of 32 rows.
    MLA_LDS char* ostage = lds + Cfg::kTileBytes + Cfg::kRedBytes;
    if (kh == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x4_t v = {(__bf16)acc[4 * i], (__bf16)acc[4 * i + 1], (__bf16)acc[4 * i + 2],
                            (__bf16)acc[4 * i + 3]};
        *reinterpret_cast<MLA_LDS bf16x4_t*>(ostage + (l & 31) * Cfg::kOutPitch +
                                             (nb * 32 + 8 * i + 4 * (l >> 5)) * 2) = v;
      }
    }
    lds_barrier();
    constexpr int kRowChunks = NT / 8;
#pragma unroll
    for (int c = tid; c < 32 * kRowChunks; c += 256) {
      const int r = c / kRowChunks, cc = c % kRowChunks;
      if (tb + r < T) {
        const u32x4_t v = *reinterpret_cast<const MLA_LDS u32x4_t*>(ostage + r * Cfg::kOutPitch + cc * 16);
        *reinterpret_cast<u32x4_t*>(C + (tb + r) * c_st + h * c_sh + n0 + cc * 8) = v;
      }
    }
    lds_barrier();                                      // staging free for the next token block
    if (more) {
      stage_act();                                      // every wave's fragment reads ended above
      lds_barrier();
    }
  }
}

// mla_up_v with the output quantized to fp8 in groups of QG (64 or 128) consecutive
// elements of a token, one float32 scale per group ([vLLM-MLA] §QuantKey: the W_UV
// output is quantized per token group of 128 or 64 when the next layer wants fp8).
// The bf16 result is formed exactly as mla_up_v forms it (float32 accumulation, one
// rounding to bf16) and then quantized: s = amax / 448, code = e4m3(x / s).
// grid = (NN / QG, N heads, token blocks of 32); a workgroup computes its group's
// 64-column sub-tiles one after the other (the W tile is staged in LDS per sub-tile
// as in head_gemm_kernel), keeps the bf16 tile in LDS, then quantizes whole groups.
// mla_up_v_fp8 launches it for QG = 64 (one sub-tile); groups of 128 go to
// up_v_fp8_g128_kernel below, which streams W instead of staging it twice.
template <int QG>
__global__ __launch_bounds__(256) void up_v_fp8_kernel(
    const uint16_t* __restrict__ A, int64_t a_st, int64_t a_sh,      // o_lat [T, N, 512]
    const uint16_t* __restrict__ W,                                   // W_UV [N, 512, 128]
    uint8_t* __restrict__ Q, int64_t q_st,                            // codes [T, N * 128]
    float* __restrict__ S, int64_t s_st,                              // scales [T, N * 128 / QG]
    int64_t T) {
  constexpr int KK = 512, NN = 128, NT = 64, KSPLIT = 2;
  using Cfg = GemmCfg<KK, NN, NT, KSPLIT>;
  constexpr int kOutPitch = QG * 2 + 16;
  __shared__ __attribute__((aligned(16))) char smem[Cfg::kTileBytes + Cfg::kRedBytes + 32 * kOutPitch +
                                                    Cfg::kABytes];
  MLA_LDS char* lds = (MLA_LDS char*)(smem);
  MLA_LDS char* ostage = lds + Cfg::kTileBytes + Cfg::kRedBytes;
  MLA_LDS char* astage = ostage + 32 * kOutPitch;

  const int h = blockIdx.y;
  const int64_t tb = (int64_t)blockIdx.z * 32;
  const int tid = threadIdx.x;
  const int w = wave_id();
  const int l = lane_id();
  const int nb = w % Cfg::kNB, kh = w / Cfg::kNB;
  const int g = l >> 4, lg = l & 15;
  const uint32_t tr_col = (uint32_t)((nb * 32 + 16 * (g & 1) + 4 * (lg & 3)) * 2);
  const int tr_row0 = 8 * (g >> 1) + (lg >> 2);
  constexpr int kChunksPerRow = NT / 8;
  constexpr int kPerThread = KK * kChunksPerRow / 256;

  // this token block's activations, read a token row at a time (whole cache lines)
  // and staged in LDS for the sub-tiles' fragment reads
  u32x4_t av[Cfg::kAPerThread];
#pragma unroll
  for (int j = 0; j < Cfg::kAPerThread; ++j) {
    const int i = tid + 256 * j;
    const int64_t t = tb + i / (KK / 8);
    av[j] = t < T ? *reinterpret_cast<const u32x4_t*>(A + t * a_st + h * a_sh + (i % (KK / 8)) * 8)
                  : u32x4_t{0u, 0u, 0u, 0u};
  }
#pragma unroll 1
  for (int sub = 0; sub < QG / NT; ++sub) {
    const int n0 = blockIdx.x * QG + sub * NT;
    const uint16_t* wh = W + (int64_t)h * KK * NN + n0;
    u32x4_t wv[kPerThread];
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int i = tid + 256 * j;
      wv[j] = *reinterpret_cast<const u32x4_t*>(wh + (int64_t)(i / kChunksPerRow) * NN + (i % kChunksPerRow) * 8);
    }
    if (sub > 0) lds_barrier();                          // the previous sub-tile's W reads are done
    if (sub == 0) {
#pragma unroll
      for (int j = 0; j < Cfg::kAPerThread; ++j) {
        const int i = tid + 256 * j;
        *reinterpret_cast<MLA_LDS u32x4_t*>(astage + (i / (KK / 8)) * Cfg::kAPitch + (i % (KK / 8)) * 16) = av[j];
      }
    }
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int i = tid + 256 * j;
      *reinterpret_cast<MLA_LDS u32x4_t*>(lds + (i / kChunksPerRow) * Cfg::kRowBytes + (i % kChunksPerRow) * 16) = wv[j];
    }
    lds_barrier();
    f32x16_t acc = {};
#pragma unroll
    for (int ks = 0; ks < Cfg::kKSteps; ++ks) {
      const int k0 = kh * Cfg::kKPerWave + ks * 16;
      const uint32_t r0 = (uint32_t)((k0 + tr_row0) * Cfg::kRowBytes) + tr_col;
      const bf16x4_t lo = lds_read_tr16(lds, r0);
      const bf16x4_t hi = lds_read_tr16(lds, r0 + 4 * Cfg::kRowBytes);
      const bf16x8_t a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const bf16x8_t b = *reinterpret_cast<const MLA_LDS bf16x8_t*>(astage + (l & 31) * Cfg::kAPitch +
                                                                     (k0 + 8 * (l >> 5)) * 2);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
    }
    MLA_LDS float* red = reinterpret_cast<MLA_LDS float*>(lds + Cfg::kTileBytes);
    if (kh == 1) {
#pragma unroll
      for (int i = 0; i < 16; ++i) red[(nb * 16 + i) * 64 + l] = acc[i];
    }
    lds_barrier();
    if (kh == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] += red[(nb * 16 + i) * 64 + l];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x4_t v = {(__bf16)acc[4 * i], (__bf16)acc[4 * i + 1], (__bf16)acc[4 * i + 2],
                            (__bf16)acc[4 * i + 3]};
        *reinterpret_cast<MLA_LDS bf16x4_t*>(ostage + (l & 31) * kOutPitch +
                                             (sub * NT + nb * 32 + 8 * i + 4 * (l >> 5)) * 2) = v;
      }
    }
  }
  lds_barrier();
  // quantize: each group is QG / 8 consecutive lanes, 8 values per lane
  constexpr int kLanesPerGroup = QG / 8;
#pragma unroll
  for (int j = 0; j < QG / 64; ++j) {
    const int item = tid + 256 * j;
    const int r = item / kLanesPerGroup, cc = item % kLanesPerGroup;
    const bool ok = tb + r < T;
    const u32x4_t raw = *reinterpret_cast<const MLA_LDS u32x4_t*>(ostage + r * kOutPitch + cc * 16);
    float x[8];
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = bf16_bits_to_f32(raw[k] & 0xFFFFu);
      x[2 * k + 1] = bf16_bits_to_f32(raw[k] >> 16);
      amax = fmaxf(amax, fmaxf(fabsf(x[2 * k]), fabsf(x[2 * k + 1])));
    }
#pragma unroll
    for (int m = 1; m < kLanesPerGroup; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
    float s = __fdiv_rn(amax, 448.0f);
    if (s == 0.f) s = 1.0f;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      lo |= e4m3_encode(__fdiv_rn(x[k], s)) << (8 * k);
      hi |= e4m3_encode(__fdiv_rn(x[4 + k], s)) << (8 * k);
    }
    if (ok) {
      const int64_t col = (int64_t)h * NN + blockIdx.x * QG + cc * 8;
      *reinterpret_cast<u32x2_t*>(Q + (tb + r) * q_st + col) = u32x2_t{lo, hi};
      if (cc == 0) S[(tb + r) * s_st + (h * NN + blockIdx.x * QG) / QG] = s;
    }
  }
}

// mla_up_v_fp8 for groups of 128: a group is a head's whole V row, so one workgroup
// owns all 128 output columns of a head for one 32-token block (wave w: columns
// 32w .. 32w+31, full K).  W_UV[h] (128 KB) streams through two LDS buffers in
// chunks of 64 k-rows, the next chunk's loads in flight while the current one is
// multiplied; the activations are staged once.  Products over k < 256 and k >= 256
// go to two accumulators that are added at the end, the order mla_up_v's K split
// uses, so the bf16 values are the ones mla_up_v writes.
__global__ __launch_bounds__(256) void up_v_fp8_g128_kernel(
    const uint16_t* __restrict__ A, int64_t a_st, int64_t a_sh,      // o_lat [T, N, 512]
    const uint16_t* __restrict__ W,                                   // W_UV [N, 512, 128]
    uint8_t* __restrict__ Q, int64_t q_st,                            // codes [T, N * 128]
    float* __restrict__ S, int64_t s_st,                              // scales [T, N]
    int64_t T) {
  constexpr int KK = 512, NN = 128, KC = 64, NCH = KK / KC;
  constexpr int kRowBytes = NN * 2 + 32;                // padded W row, as in the absorb tile
  constexpr int kBufBytes = KC * kRowBytes;
  constexpr int kAPitch = KK * 2 + 16;
  constexpr int kOutPitch = NN * 2 + 16;
  constexpr int kWPerThread = KC * (NN / 8) / 256;      // 4 chunks of 16 B
  constexpr int kAPerThread = 32 * KK / 8 / 256;        // 8
  __shared__ __attribute__((aligned(16))) char smem[2 * kBufBytes + 32 * kAPitch + 32 * kOutPitch];
  MLA_LDS char* lds = (MLA_LDS char*)(smem);
  MLA_LDS char* astage = lds + 2 * kBufBytes;
  MLA_LDS char* ostage = astage + 32 * kAPitch;

  const int h = blockIdx.y;
  const int64_t tb = (int64_t)blockIdx.z * 32;
  const int tid = threadIdx.x;
  const int nb = wave_id();
  const int l = lane_id();
  const int g = l >> 4, lg = l & 15;
  const uint32_t tr_col = (uint32_t)((nb * 32 + 16 * (g & 1) + 4 * (lg & 3)) * 2);
  const int tr_row0 = 8 * (g >> 1) + (lg >> 2);
  const uint16_t* wh = W + (int64_t)h * KK * NN;

  u32x4_t av[kAPerThread], wv[2][kWPerThread];      // two chunks of W in flight
#pragma unroll
  for (int j = 0; j < kAPerThread; ++j) {
    const int i = tid + 256 * j;
    const int64_t t = tb + i / (KK / 8);
    av[j] = t < T ? *reinterpret_cast<const u32x4_t*>(A + t * a_st + h * a_sh + (i % (KK / 8)) * 8)
                  : u32x4_t{0u, 0u, 0u, 0u};
  }
  auto load_w = [&](int kc, u32x4_t (&r)[kWPerThread]) {
#pragma unroll
    for (int j = 0; j < kWPerThread; ++j) {
      const int i = tid + 256 * j;
      r[j] = *reinterpret_cast<const u32x4_t*>(wh + (int64_t)(kc * KC + i / (NN / 8)) * NN + (i % (NN / 8)) * 8);
    }
  };
  auto store_w = [&](int buf, const u32x4_t (&r)[kWPerThread]) {
#pragma unroll
    for (int j = 0; j < kWPerThread; ++j) {
      const int i = tid + 256 * j;
      *reinterpret_cast<MLA_LDS u32x4_t*>(lds + buf * kBufBytes + (i / (NN / 8)) * kRowBytes + (i % (NN / 8)) * 16) =
          r[j];
    }
  };
  load_w(0, wv[0]);
  load_w(1, wv[1]);
#pragma unroll
  for (int j = 0; j < kAPerThread; ++j) {
    const int i = tid + 256 * j;
    *reinterpret_cast<MLA_LDS u32x4_t*>(astage + (i / (KK / 8)) * kAPitch + (i % (KK / 8)) * 16) = av[j];
  }
  store_w(0, wv[0]);
  lds_barrier();

  // chunk kc + 2 is requested while chunk kc is multiplied and chunk kc + 1 (requested
  // one step earlier) goes into the other LDS buffer
  f32x16_t acc_lo = {}, acc_hi = {};
#pragma unroll
  for (int kc = 0; kc < NCH; ++kc) {
    if (kc + 2 < NCH) load_w(kc + 2, wv[kc & 1]);     // chunk kc's registers were stored last step
    f32x16_t& acc = kc < NCH / 2 ? acc_lo : acc_hi;
    const uint32_t base = (uint32_t)((kc & 1) * kBufBytes);
#pragma unroll
    for (int ks = 0; ks < KC / 16; ++ks) {
      const uint32_t r0 = base + (uint32_t)((ks * 16 + tr_row0) * kRowBytes) + tr_col;
      const bf16x4_t lo = lds_read_tr16(lds, r0);
      const bf16x4_t hi = lds_read_tr16(lds, r0 + 4 * kRowBytes);
      const bf16x8_t a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const bf16x8_t b = *reinterpret_cast<const MLA_LDS bf16x8_t*>(
          astage + (l & 31) * kAPitch + (kc * KC + ks * 16 + 8 * (l >> 5)) * 2);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
    }
    if (kc + 1 < NCH) {
      store_w((kc + 1) & 1, wv[(kc + 1) & 1]);          // that buffer's last reader was chunk kc - 1
      lds_barrier();
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float y0 = acc_lo[4 * i] + acc_hi[4 * i], y1 = acc_lo[4 * i + 1] + acc_hi[4 * i + 1];
    const float y2 = acc_lo[4 * i + 2] + acc_hi[4 * i + 2], y3 = acc_lo[4 * i + 3] + acc_hi[4 * i + 3];
    const bf16x4_t v = {(__bf16)y0, (__bf16)y1, (__bf16)y2, (__bf16)y3};
    *reinterpret_cast<MLA_LDS bf16x4_t*>(ostage + (l & 31) * kOutPitch + (nb * 32 + 8 * i + 4 * (l >> 5)) * 2) = v;
  }
  lds_barrier();
  // quantize: a token's group is 16 consecutive lanes of 8 values
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int item = tid + 256 * j;
    const int r = item / 16, cc = item % 16;
    const u32x4_t raw = *reinterpret_cast<const MLA_LDS u32x4_t*>(ostage + r * kOutPitch + cc * 16);
    float x[8];
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = bf16_bits_to_f32(raw[k] & 0xFFFFu);
      x[2 * k + 1] = bf16_bits_to_f32(raw[k] >> 16);
      amax = fmaxf(amax, fmaxf(fabsf(x[2 * k]), fabsf(x[2 * k + 1])));
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
    float sc = __fdiv_rn(amax, 448.0f);
    if (sc == 0.f) sc = 1.0f;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      lo |= e4m3_encode(__fdiv_rn(x[k], sc)) << (8 * k);
      hi |= e4m3_encode(__fdiv_rn(x[4 + k], sc)) << (8 * k);
    }
    if (tb + r < T) {
      *reinterpret_cast<u32x2_t*>(Q + (tb + r) * q_st + (int64_t)h * NN + cc * 8) = u32x2_t{lo, hi};
      if (cc == 0) S[(tb + r) * s_st + h] = sc;
    }
  }
}

// When the up-projections take head_gemm_stream_kernel and with how many workgroups per
// CU, from sweeps of T with 128 heads and cold weights (8 rotating copies):
//  * up_v from T = 128 (T = 64: 9.0 us for the tile kernel against 10.6), one workgroup
//    per CU at every size measured (each workgroup loads its head's weights once, so
//    fewer workgroups load them fewer times: T = 4096 118.9 against 132.1 us with two,
//    T = 8192 227 against 251);
//  * up_v_fp8 with groups of 128 from T = 192 (the tile kernel 12.3 against 14.0 us at
//    128), one workgroup per CU below T = 1024 (T = 512: 26.8 against 29.3 us) and two
//    from 1024, where the second workgroup's waves hide the quantizing epilogue (T = 4096:
//    133.9 against 149.0 us);
//  * kv_b_proj from S = 128 (22.3 us for the tile kernel against 14.2), one workgroup per
//    CU below S = 512 and two from 512, where the MFMA work needs the second workgroup's
//    waves (S = 4096: 144.9 against 169.4 us).
constexpr int64_t kUpvStreamMinT = 128;
constexpr int64_t kUpvFp8StreamMinT = 192;
constexpr int64_t kUpvFp8TwoPerCuMinT = 1024;
constexpr int64_t kKvbStreamMinS = 128;
constexpr int64_t kKvbTwoPerCuMinS = 512;

// ---------------------------------------------------------------------------
// Head GEMM for many tokens, weight-stationary form (mla_up_v, mla_up_v_fp8 with groups of
// 128, mla_kv_b_proj): C[t, h, n0 : n0+128] = A[t, h, 0:512] . W[h][0:512][n0 : n0+128].
// A workgroup of four waves owns one head, one 128-column half and a contiguous range of
// 16-token stages; grid = (parts, heads, NN / 128), one or two workgroups per CU.  Each
// wave keeps the weights of its 32 columns over all of K = 512 in registers (the MFMA
// A operand of two 16x16x32 products per 32 k, 128 VGPRs), loaded once through LDS in
// two halves with transpose reads, so the weights leave HBM once per workgroup instead
// of once per token tile.  The token rows then stream through a ring of four LDS slots:
// one global->LDS copy per row moves a token's whole 1 KiB (512 bf16) of this head in one
// instruction, rows padded to 1056 B (with 1040 B the fragment reads measured about five
// times the bank conflicts).  One barrier per stage: after it, the copy of stage c + 3
// goes into the slot stage c - 1 has left, the tile of stage c - 1 leaves from one of two
// LDS staging buffers, and stage c is multiplied into the other.  Tiles leave as whole
// row segments (bf16) or quantized per token (fp8 codes in groups of the 128 columns, one
// float32 scale), with nontemporal stores (the outputs are not read again by this call).
// Rows past T are copied from row T - 1 and never stored, so every wave issues the same
// number of copies per stage and the vmcnt values below are exact.  About 75 KB of LDS.
// ---------------------------------------------------------------------------
constexpr int kHsTok = 16;                                   // tokens per stage
constexpr int kHsSlots = 4;                                  // ring slots (3 stages ahead)
constexpr int kHsRowPitch = 1024 + 32;                       // one token's 512 bf16, padded
constexpr int kHsSlot = kHsTok * kHsRowPitch;                // 16896
constexpr int kHsOutPitch = 128 * 2 + 16;                    // 272
constexpr int kHsOutBytes = kHsTok * kHsOutPitch;            // one staging buffer
constexpr int kHsOut = kHsSlots * kHsSlot;                   // two staging buffers from here
constexpr int kHsLds = kHsOut + 2 * kHsOutBytes;             // 76288
constexpr int kHsCopies = kHsTok / 4;                        // row copies per wave and stage
static_assert(kHsSlots * kHsSlot >= 256 * 256, "half of a head's weights fits the ring for the transpose pass");
static_assert(kHsTok * 16 == 256, "the epilogue gives one 16-byte chunk to each thread");

__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t u = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}

// e4m3fn codes of four float32 values already within [-448, 448] (round to nearest even,
// subnormals kept): the same codes as e4m3_encode, by the conversion instruction
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  return (uint32_t)v;
}

// One 1 KiB global->LDS row copy as dma_16B<0, 0>, marked nontemporal: for activations
// that are read exactly once, so their lines go first when the caches need room
__device__ __forceinline__ void dma_16B_nt(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile(
      "s_add_u32 m0, %2, 0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1 offset:0 nt"
      :
      : "v"(voff), "s"(sbase), "s"(lds_base)
      : "memory", "scc");
}

// STREAM_A: every activation row is read by one workgroup only (a head's own rows), so
// the copies are nontemporal; the shared latent rows of kv_b_proj are read by every head
// and stay cacheable.
template <bool FP8OUT, bool STREAM_A>
__global__ __launch_bounds__(256, 2) void head_gemm_stream_kernel(
    const uint16_t* __restrict__ A, int64_t a_st, int64_t a_sh,      // [T, N or shared, 512]
    const uint16_t* __restrict__ W, int nn,                           // [N, 512, nn]
    uint16_t* __restrict__ C, int64_t c_st, int64_t c_sh,            // bf16 [T, N, nn]
    uint8_t* __restrict__ Q, int64_t q_st,                            // fp8 codes [T, N * 128]
    float* __restrict__ S, int64_t s_st,                              // scales [T, N]
    int64_t T, int parts) {
  __shared__ __attribute__((aligned(16))) char smem[kHsLds];
  MLA_LDS char* lds = (MLA_LDS char*)(smem);
  const uint32_t lbase = (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr(lds));
  const int h = blockIdx.y;
  const int n0 = blockIdx.z * 128;
  const int tid = threadIdx.x;
  const int w = wave_id();
  const int l = lane_id();
  const int g = l >> 4, lg = l & 15;
  const int64_t chunks = (T + kHsTok - 1) / kHsTok;
  const int64_t c0 = chunks * blockIdx.x / parts, c1 = chunks * (blockIdx.x + 1) / parts;

  // weights: two passes of 256 k rows x 128 columns (256 B per row, unpadded: a copy
  // instruction fills four rows), read back transposed into the MFMA A operand: for
  // column half c and step s, lane l holds column 32 w + 16 c + (l & 15) and k rows
  // 32 s + 8 (l >> 4) + 0..7
  bf16x8_t wf[2][16];
  const char* wsrc = reinterpret_cast<const char*>(W + (int64_t)h * 512 * nn + n0);
  const uint32_t wvoff = (uint32_t)((l >> 4) * nn * 2 + (l & 15) * 16);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int i = w * 16 + j;                          // rows 4 i .. 4 i + 3 of the pass
      dma_16B<0, 0>(uniform_ptr(wsrc + (int64_t)(256 * q + 4 * i) * nn * 2), wvoff, lbase + 1024 * i);
    }
    wait_vmcnt<0>();
    lds_barrier();
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint32_t r0 = lbase + (uint32_t)((32 * s + 8 * g + (lg >> 2)) * 256 + (32 * w + 16 * c + 4 * (lg & 3)) * 2);
        const bf16x4_t lo = lds_read_tr16_at(r0);
        const bf16x4_t hi = lds_read_tr16_at(r0 + 4 * 256);
        wf[c][8 * q + s] = bf16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    lds_barrier();
  }

  const char* asrc = reinterpret_cast<const char*>(A + (int64_t)h * a_sh);
  const uint32_t avoff = (uint32_t)(l * 16);
  // the copies of one stage: wave w moves rows 4 w .. 4 w + 3 (token rows past T repeat
  // row T - 1; their products are not stored)
  auto issue = [&](int64_t ci) {
    const int64_t tb = ci * kHsTok;
    const int slot = (int)((ci - c0) % kHsSlots);
#pragma unroll
    for (int j = 0; j < kHsCopies; ++j) {
      const int r = w * kHsCopies + j;
      const int64_t t = tb + r < T ? tb + r : T - 1;
      const uint32_t dst = (uint32_t)__builtin_amdgcn_readfirstlane(lbase + slot * kHsSlot + r * kHsRowPitch);
      if constexpr (STREAM_A)
        dma_16B_nt(uniform_ptr(asrc + t * a_st * 2), avoff, dst);
      else
        dma_16B<0, 0>(uniform_ptr(asrc + t * a_st * 2), avoff, dst);
    }
  };

  // activation fragments (B operand): token l & 15 of the stage, k 32 s + 8 (l >> 4)
  const uint32_t bread = lbase + (uint32_t)((l & 15) * kHsRowPitch + 16 * (l >> 4));
  const int r = tid / 16, cc = tid % 16;                 // epilogue: token row, 16-byte chunk

  // the finished tile of stage ci leaves from staging buffer ci & 1 one stage later
  auto epilogue = [&](int64_t ci) {
    const MLA_LDS char* ostage = lds + kHsOut + (int)(ci & 1) * kHsOutBytes;
    const int64_t tb = ci * kHsTok;
    if constexpr (!FP8OUT) {
      if (tb + r < T) {
        const u32x4_t v = *reinterpret_cast<const MLA_LDS u32x4_t*>(ostage + r * kHsOutPitch + cc * 16);
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(C + (tb + r) * c_st + (int64_t)h * c_sh + n0 + cc * 8));
      }
    } else {
      // a token's group of 128 values is 16 consecutive lanes of 8 values
      const u32x4_t raw = *reinterpret_cast<const MLA_LDS u32x4_t*>(ostage + r * kHsOutPitch + cc * 16);
      float x[8];
      float amax = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[2 * k] = bf16_bits_to_f32(raw[k] & 0xFFFFu);
        x[2 * k + 1] = bf16_bits_to_f32(raw[k] >> 16);
        amax = fmaxf(amax, fmaxf(fabsf(x[2 * k]), fabsf(x[2 * k + 1])));
      }
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
      float sc = __fdiv_rn(amax, 448.0f);
      if (sc == 0.f) sc = 1.0f;
      // |x / sc| <= 448 (1 + 2^-23) after rounding: clamping to 448 keeps every code
      float y[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) y[k] = fminf(fmaxf(__fdiv_rn(x[k], sc), -448.0f), 448.0f);
      const uint32_t lo = e4m3_pack4(y[0], y[1], y[2], y[3]);
      const uint32_t hi = e4m3_pack4(y[4], y[5], y[6], y[7]);
      if (tb + r < T) {
        __builtin_nontemporal_store(u32x2_t{lo, hi},
                                    reinterpret_cast<u32x2_t*>(Q + (tb + r) * q_st + (int64_t)h * 128 + cc * 8));
        if (cc == 0) S[(tb + r) * s_st + h] = sc;
      }
    }
  };

#pragma unroll
  for (int k = 0; k < kHsSlots - 1; ++k)
    if (c0 + k < c1) issue(c0 + k);
#pragma unroll 1
  for (int64_t ci = c0; ci < c1; ++ci) {
    // wait for this stage's copies: the newer ones in flight are those of the next
    // min(2, c1 - 1 - ci) stages (stores of earlier stages may finish in any order; the
    // count covers copies only, which complete in order)
    const int64_t ahead = c1 - 1 - ci;
    if (ahead >= 2) wait_vmcnt<2 * kHsCopies>();
    else if (ahead == 1) wait_vmcnt<kHsCopies>();
    else wait_vmcnt<0>();
    // one barrier per stage: stage ci landed for every wave; stage ci - 1's slot has been
    // read by every wave, and its tile staged
    lds_barrier();
    if (ci + kHsSlots - 1 < c1) issue(ci + kHsSlots - 1);   // into the slot of stage ci - 1
    if (ci > c0) epilogue(ci - 1);
    f32x4_t acc[2] = {};
    const uint32_t b0 = bread + (uint32_t)(((ci - c0) % kHsSlots) * kHsSlot);
    // fragment reads run four steps ahead of the products (the scheduler would otherwise
    // pull each read down next to its use)
    bf16x8_t x[16];
#pragma unroll
    for (int s = 0; s < 4; ++s) x[s] = lds_read_b128_at(b0 + 64 * s);
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      if (s + 4 < 16) x[s + 4] = lds_read_b128_at(b0 + 64 * (s + 4));
      __builtin_amdgcn_sched_barrier(0);
      acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[0][s], x[s], acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[1][s], x[s], acc[1], 0, 0, 0);
    }
    // lane (l & 15) is token l & 15 of the stage, columns 32 w + 16 c + 4 (l >> 4) + 0..3;
    // staging buffer ci & 1 was last read by the epilogue of stage ci - 2, before the barrier
    MLA_LDS char* ostage = lds + kHsOut + (int)(ci & 1) * kHsOutBytes;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bf16x4_t v = {(__bf16)acc[c][0], (__bf16)acc[c][1], (__bf16)acc[c][2], (__bf16)acc[c][3]};
      *reinterpret_cast<MLA_LDS bf16x4_t*>(ostage + (l & 15) * kHsOutPitch + (32 * w + 16 * c + 4 * (l >> 4)) * 2) = v;
    }
  }
  if (c0 < c1) {
    lds_barrier();                                       // the last tile is staged
    epilogue(c1 - 1);
  }
}

// workgroups per (head, column half) of head_gemm_stream_kernel: about per_cu of them per
// CU over the grid, never more than the 16-token stages
static int stream_parts(int64_t T, int units, int cu_count, int per_cu) {
  const int64_t stages = (T + kHsTok - 1) / kHsTok;
  int64_t p = ((int64_t)per_cu * (cu_count > 0 ? cu_count : 256) + units - 1) / units;
  if (p > stages) p = stages;
  return (int)(p < 1 ? 1 : p);
}

}  // namespace mla

extern "C" mla_status_t mla_absorb_q(const void* q_nope, int64_t qn_stride_t, int64_t qn_stride_h,
                                     const void* q_pe, int64_t qp_stride_t, int64_t qp_stride_h,
                                     const void* w_uk_t, int64_t T, int32_t N, void* q_fused,
                                     int64_t qf_stride_t, int64_t qf_stride_h, void* stream) {
  using namespace mla;
  if (T < 0 || N < 1 || N > MLA_MAX_HEADS) return MLA_ERR_SHAPE;
  if (T == 0) return MLA_OK;
  if (!q_nope || !w_uk_t || !q_fused) return MLA_ERR_NULL;
  if (!aligned16(q_nope) || !aligned16(w_uk_t) || !aligned16(q_fused) || !mult8(qn_stride_t) ||
      !mult8(qn_stride_h) || !mult8(qf_stride_t) || !mult8(qf_stride_h))
    return MLA_ERR_ALIGN;
  if (q_pe && (!aligned16(q_pe) || !mult8(qp_stride_t) || !mult8(qp_stride_h))) return MLA_ERR_ALIGN;
  DeviceInfo di;
  mla_status_t st = device_info(&di);
  if (st != MLA_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  dim3 grid(MLA_KV_LORA_RANK / 128, N);
  if (q_pe)
    hipLaunchKernelGGL((head_gemm_kernel<128, 512, 128, 1, kCopyTail>), grid, dim3(256), 0, s,
                       (const uint16_t*)q_nope, qn_stride_t, qn_stride_h, (const uint16_t*)w_uk_t,
                       (uint16_t*)q_fused, qf_stride_t, qf_stride_h, (const uint16_t*)q_pe,
                       qp_stride_t, qp_stride_h, (const int64_t*)nullptr, (const float*)nullptr,
                       (int64_t)0, 0, T, CacheRowsArgs{});
  else
    hipLaunchKernelGGL((head_gemm_kernel<128, 512, 128, 1, kNoTail>), grid, dim3(256), 0, s,
                       (const uint16_t*)q_nope, qn_stride_t, qn_stride_h, (const uint16_t*)w_uk_t,
                       (uint16_t*)q_fused, qf_stride_t, qf_stride_h, (const uint16_t*)nullptr,
                       (int64_t)0, (int64_t)0, (const int64_t*)nullptr, (const float*)nullptr,
                       (int64_t)0, 0, T, CacheRowsArgs{});
  return launch_status();
}

// mla_absorb_q and mla_cache_write in one launch: the cache-row workgroups (four tokens
// each) take the first rows of the absorption grid, so the step's two smallest kernels
// cost one launch.  The arguments and checks are those of the two calls.
extern "C" mla_status_t mla_absorb_q_cache_write(const void* q_nope, int64_t qn_stride_t, int64_t qn_stride_h,
                                                 const void* q_pe, int64_t qp_stride_t, int64_t qp_stride_h,
                                                 const void* w_uk_t, int64_t T, int32_t N, void* q_fused,
                                                 int64_t qf_stride_t, int64_t qf_stride_h, const void* kv_c,
                                                 int64_t kv_c_stride_t, const void* k_pe, int64_t k_pe_stride_t,
                                                 const int64_t* slot_mapping, int64_t T_new, void* kv_cache,
                                                 int32_t kv_dtype, int64_t num_pages, void* stream) {
  using namespace mla;
  if (T < 0 || N < 1 || N > MLA_MAX_HEADS) return MLA_ERR_SHAPE;
  if (T == 0) return mla_cache_write(kv_c, kv_c_stride_t, k_pe, k_pe_stride_t, slot_mapping, T_new, kv_cache,
                                     kv_dtype, num_pages, stream);
  if (!q_nope || !w_uk_t || !q_fused) return MLA_ERR_NULL;
  if (!aligned16(q_nope) || !aligned16(w_uk_t) || !aligned16(q_fused) || !mult8(qn_stride_t) ||
      !mult8(qn_stride_h) || !mult8(qf_stride_t) || !mult8(qf_stride_h))
    return MLA_ERR_ALIGN;
  if (q_pe && (!aligned16(q_pe) || !mult8(qp_stride_t) || !mult8(qp_stride_h))) return MLA_ERR_ALIGN;
  const mla_status_t cst = cache_write_check(kv_c, kv_c_stride_t, k_pe, k_pe_stride_t, slot_mapping, T_new,
                                             kv_cache, kv_dtype, num_pages);
  if (cst != MLA_OK) return cst;
  const int64_t row_wgs = (T_new + 3) / 4;               // four tokens per workgroup
  const int64_t row_lines = (row_wgs + 3) / 4;           // four workgroups per grid row
  if ((int64_t)N + row_lines > 65535) return MLA_ERR_SHAPE;
  DeviceInfo di;
  mla_status_t st = device_info(&di);
  if (st != MLA_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const CacheRowsArgs cw{(const uint16_t*)kv_c, kv_c_stride_t, (const uint16_t*)k_pe, k_pe_stride_t,
                         slot_mapping, T_new, (char*)kv_cache, num_pages, (int32_t)row_lines};
  dim3 grid(MLA_KV_LORA_RANK / 128, (unsigned)(N + row_lines));
  auto go = [&](auto pe_c, auto cw_c) {
    constexpr int PE = decltype(pe_c)::value, CW = decltype(cw_c)::value;
    hipLaunchKernelGGL((head_gemm_kernel<128, 512, 128, 1, PE, CW>), grid, dim3(256), 0, s,
                       (const uint16_t*)q_nope, qn_stride_t, qn_stride_h, (const uint16_t*)w_uk_t,
                       (uint16_t*)q_fused, qf_stride_t, qf_stride_h, (const uint16_t*)q_pe, qp_stride_t,
                       qp_stride_h, (const int64_t*)nullptr, (const float*)nullptr, (int64_t)0, 0, T, cw);
  };
  const bool fp8 = kv_dtype == MLA_KV_FP8_E4M3;
  if (q_pe) {
    if (fp8) go(std::integral_constant<int, kCopyTail>{}, std::integral_constant<int, kRowsFp8>{});
    else go(std::integral_constant<int, kCopyTail>{}, std::integral_constant<int, kRowsBf16>{});
  } else {
    if (fp8) go(std::integral_constant<int, kNoTail>{}, std::integral_constant<int, kRowsFp8>{});
    else go(std::integral_constant<int, kNoTail>{}, std::integral_constant<int, kRowsBf16>{});
  }
  return launch_status();
}

extern "C" mla_status_t mla_absorb_q_rope(const void* q_nope, int64_t qn_stride_t, int64_t qn_stride_h,
                                          const void* q_pe, int64_t qp_stride_t, int64_t qp_stride_h,
                                          const void* w_uk_t, int64_t T, int32_t N, const int64_t* positions,
                                          const float* cos_sin_cache, int64_t max_pos, int32_t neox,
                                          void* q_fused, int64_t qf_stride_t, int64_t qf_stride_h,
                                          void* stream) {
  using namespace mla;
  if (T < 0 || N < 1 || N > MLA_MAX_HEADS || max_pos < 1) return MLA_ERR_SHAPE;
  if (T == 0) return MLA_OK;
  if (!q_nope || !w_uk_t || !q_fused || !q_pe || !positions || !cos_sin_cache) return MLA_ERR_NULL;
  if (!aligned16(q_nope) || !aligned16(w_uk_t) || !aligned16(q_fused) || !mult8(qn_stride_t) ||
      !mult8(qn_stride_h) || !mult8(qf_stride_t) || !mult8(qf_stride_h) || !aligned16(q_pe) ||
      !mult8(qp_stride_t) || !mult8(qp_stride_h) || !aligned16(cos_sin_cache) ||
      (reinterpret_cast<uintptr_t>(positions) & 7u))
    return MLA_ERR_ALIGN;
  DeviceInfo di;
  mla_status_t st = device_info(&di);
  if (st != MLA_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  dim3 grid(MLA_KV_LORA_RANK / 128, N);
  hipLaunchKernelGGL((head_gemm_kernel<128, 512, 128, 1, kRopeTail>), grid, dim3(256), 0, s,
                     (const uint16_t*)q_nope, qn_stride_t, qn_stride_h, (const uint16_t*)w_uk_t,
                     (uint16_t*)q_fused, qf_stride_t, qf_stride_h, (const uint16_t*)q_pe, qp_stride_t,
                     qp_stride_h, positions, cos_sin_cache, max_pos, neox ? 1 : 0, T, CacheRowsArgs{});
  return launch_status();
}

extern "C" mla_status_t mla_up_v(const void* o_lat, int64_t ol_stride_t, int64_t ol_stride_h,
                                 const void* w_uv, int64_t T, int32_t N, void* out,
                                 int64_t out_stride_t, void* stream) {
  using namespace mla;
  if (T < 0 || N < 1 || N > MLA_MAX_HEADS) return MLA_ERR_SHAPE;
  if (T == 0) return MLA_OK;
  if (!o_lat || !w_uv || !out) return MLA_ERR_NULL;
  if (out_stride_t < (int64_t)N * MLA_V_HEAD_DIM) return MLA_ERR_SHAPE;
  if (!aligned16(o_lat) || !aligned16(w_uv) || !aligned16(out) || !mult8(ol_stride_t) ||
      !mult8(ol_stride_h) || !mult8(out_stride_t))
    return MLA_ERR_ALIGN;
  DeviceInfo di;
  mla_status_t st = device_info(&di);
  if (st != MLA_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (T >= kUpvStreamMinT) {
    const int parts = stream_parts(T, N, di.cu_count, 1);
    hipLaunchKernelGGL((head_gemm_stream_kernel<false, true>), dim3((unsigned)parts, N, 1), dim3(256), 0, s,
                       (const uint16_t*)o_lat, ol_stride_t, ol_stride_h, (const uint16_t*)w_uv, MLA_V_HEAD_DIM,
                       (uint16_t*)out, out_stride_t, (int64_t)MLA_V_HEAD_DIM, (uint8_t*)nullptr, (int64_t)0,
                       (float*)nullptr, (int64_t)0, T, parts);
    return launch_status();
  }
  dim3 grid(MLA_V_HEAD_DIM / 64, N);
  hipLaunchKernelGGL((head_gemm_kernel<512, 128, 64, 2, kNoTail>), grid, dim3(256), 0, s,
                     (const uint16_t*)o_lat, ol_stride_t, ol_stride_h, (const uint16_t*)w_uv,
                     (uint16_t*)out, out_stride_t, (int64_t)MLA_V_HEAD_DIM,
                     (const uint16_t*)nullptr, (int64_t)0, (int64_t)0, (const int64_t*)nullptr,
                     (const float*)nullptr, (int64_t)0, 0, T, CacheRowsArgs{});
  return launch_status();
}

extern "C" mla_status_t mla_up_v_fp8(const void* o_lat, int64_t ol_stride_t, int64_t ol_stride_h,
                                     const void* w_uv, int64_t T, int32_t N, int32_t group, void* out_codes,
                                     int64_t codes_stride_t, float* out_scales, int64_t scales_stride_t,
                                     void* stream) {
  using namespace mla;
  if (T < 0 || N < 1 || N > MLA_MAX_HEADS || (group != 64 && group != 128)) return MLA_ERR_SHAPE;
  if (T == 0) return MLA_OK;
  if (T > (int64_t)65535 * 32) return MLA_ERR_SHAPE;        // token blocks ride grid z
  if (!o_lat || !w_uv || !out_codes || !out_scales) return MLA_ERR_NULL;
  if (codes_stride_t < (int64_t)N * MLA_V_HEAD_DIM || scales_stride_t < (int64_t)N * MLA_V_HEAD_DIM / group)
    return MLA_ERR_SHAPE;
  if (!aligned16(o_lat) || !aligned16(w_uv) || !mult8(ol_stride_t) || !mult8(ol_stride_h) ||
      (reinterpret_cast<uintptr_t>(out_codes) & 7u) || (codes_stride_t & 7) ||
      (reinterpret_cast<uintptr_t>(out_scales) & 3u))
    return MLA_ERR_ALIGN;
  DeviceInfo di;
  mla_status_t st = device_info(&di);
  if (st != MLA_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)(MLA_V_HEAD_DIM / group), (unsigned)N, (unsigned)((T + 31) / 32));
  if (group == 128 && T >= kUpvFp8StreamMinT) {
    const int parts = stream_parts(T, N, di.cu_count, T >= kUpvFp8TwoPerCuMinT ? 2 : 1);
    hipLaunchKernelGGL((head_gemm_stream_kernel<true, true>), dim3((unsigned)parts, N, 1), dim3(256), 0, s,
                       (const uint16_t*)o_lat, ol_stride_t, ol_stride_h, (const uint16_t*)w_uv, MLA_V_HEAD_DIM,
                       (uint16_t*)nullptr, (int64_t)0, (int64_t)0, (uint8_t*)out_codes, codes_stride_t, out_scales,
                       scales_stride_t, T, parts);
  }
  else if (group == 64)
    hipLaunchKernelGGL(up_v_fp8_kernel<64>, grid, dim3(256), 0, s, (const uint16_t*)o_lat, ol_stride_t,
                       ol_stride_h, (const uint16_t*)w_uv, (uint8_t*)out_codes, codes_stride_t, out_scales,
                       scales_stride_t, T);
  else
    hipLaunchKernelGGL(up_v_fp8_g128_kernel, grid, dim3(256), 0, s, (const uint16_t*)o_lat, ol_stride_t,
                       ol_stride_h, (const uint16_t*)w_uv, (uint8_t*)out_codes, codes_stride_t, out_scales,
                       scales_stride_t, T);
  return launch_status();
}

extern "C" mla_status_t mla_kv_b_proj(const void* kv_c, int64_t kc_stride_t, const void* w_kvb, int64_t S,
                                      int32_t N, void* out, int64_t out_stride_t, int64_t out_stride_h,
                                      void* stream) {
  using namespace mla;
  if (S < 0 || N < 1 || N > MLA_MAX_HEADS) return MLA_ERR_SHAPE;
  if (S == 0) return MLA_OK;
  if (!kv_c || !w_kvb || !out) return MLA_ERR_NULL;
  if (!aligned16(kv_c) || !aligned16(w_kvb) || !aligned16(out) || !mult8(kc_stride_t) || !mult8(out_stride_t) ||
      !mult8(out_stride_h))
    return MLA_ERR_ALIGN;
  DeviceInfo di;
  mla_status_t st = device_info(&di);
  if (st != MLA_OK) return st;
  // the latent has no head dimension: every head's workgroups read the same rows
  if (S >= kKvbStreamMinS) {
    const int parts = stream_parts(S, 2 * N, di.cu_count, S >= kKvbTwoPerCuMinS ? 2 : 1);
    hipLaunchKernelGGL((head_gemm_stream_kernel<false, false>), dim3((unsigned)parts, N, 2), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), (const uint16_t*)kv_c, kc_stride_t, (int64_t)0,
                       (const uint16_t*)w_kvb, 256, (uint16_t*)out, out_stride_t, out_stride_h, (uint8_t*)nullptr,
                       (int64_t)0, (float*)nullptr, (int64_t)0, S, parts);
    return launch_status();
  }
  hipLaunchKernelGGL((head_gemm_kernel<512, 256, 64, 2, kNoTail>), dim3(256 / 64, N), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), (const uint16_t*)kv_c, kc_stride_t, (int64_t)0,
                     (const uint16_t*)w_kvb, (uint16_t*)out, out_stride_t, out_stride_h, (const uint16_t*)nullptr,
                     (int64_t)0, (int64_t)0, (const int64_t*)nullptr, (const float*)nullptr, (int64_t)0, 0, S,
                     CacheRowsArgs{});
  return launch_status();
}
