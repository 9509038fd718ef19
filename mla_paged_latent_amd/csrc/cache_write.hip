// mla_cache_write: concat-and-cache scatter of [kv_c | k_pe] rows into 64-token
// pages, bf16 (bit copy) or fp8 e4m3fn with a per-token float32 scale.
// Source: "vLLM 源码完全拆解(三十七):MLA 注意力后端", §写缓存 (latent and k_pe written
// into one row per token by one kernel at slot_mapping[t]) and §缓存的形状 (576-element
// rows; fp8 rows carry one float32 scale for K and one for V, 584 bytes).
#include "cache_rows.h"
#include "mla_common.h"
#include "mla_host.h"

namespace mla {

// One wave per token, four tokens per 256-thread workgroup.
template <bool FP8>
__global__ __launch_bounds__(256) void cache_write_kernel(
    const uint16_t* __restrict__ kv_c, int64_t kv_stride, const uint16_t* __restrict__ k_pe,
    int64_t pe_stride, const int64_t* __restrict__ slots, int64_t T, char* __restrict__ pool,
    int64_t num_pages) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  cache_write_row<FP8>(kv_c, kv_stride, k_pe, pe_stride, slots, pool, num_pages, t, lane_id());
}

}  // namespace mla

extern "C" mla_status_t mla_cache_write(const void* kv_c, int64_t kv_c_stride_t, const void* k_pe,
                                        int64_t k_pe_stride_t, const int64_t* slot_mapping,
                                        int64_t T, void* kv_cache, int32_t kv_dtype,
                                        int64_t num_pages, void* stream) {
  using namespace mla;
  const mla_status_t cst =
      cache_write_check(kv_c, kv_c_stride_t, k_pe, k_pe_stride_t, slot_mapping, T, kv_cache, kv_dtype, num_pages);
  if (cst != MLA_OK || T == 0) return cst;
  DeviceInfo di;
  mla_status_t st = device_info(&di);
  if (st != MLA_OK) return st;
  const int64_t blocks = (T + 3) / 4;
  if (blocks > 0x7fffffff) return MLA_ERR_SHAPE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (kv_dtype == MLA_KV_BF16)
    hipLaunchKernelGGL(cache_write_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s,
                       (const uint16_t*)kv_c, kv_c_stride_t, (const uint16_t*)k_pe, k_pe_stride_t,
                       slot_mapping, T, (char*)kv_cache, num_pages);
  else
    hipLaunchKernelGGL(cache_write_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s,
                       (const uint16_t*)kv_c, kv_c_stride_t, (const uint16_t*)k_pe, k_pe_stride_t,
                       slot_mapping, T, (char*)kv_cache, num_pages);
  return launch_status();
}

extern "C" const char* mla_status_str(mla_status_t status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL: return "MLA_ERR_NULL: a required pointer is NULL";
    case MLA_ERR_SHAPE: return "MLA_ERR_SHAPE: size outside the supported range";
    case MLA_ERR_DTYPE: return "MLA_ERR_DTYPE: unknown kv_dtype";
    case MLA_ERR_ALIGN: return "MLA_ERR_ALIGN: pointer or stride not 16-byte aligned";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace missing or too small";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: HIP runtime or launch failure";
    case MLA_ERR_DEVICE: return "MLA_ERR_DEVICE: current device is not gfx950";
  }
  return "unknown mla_status_t";
}
