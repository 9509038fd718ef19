// Measurement probes for bench.py (not part of the decode path): the achievable HBM
// read bandwidth and bf16 MFMA rate of the device, so that the decode kernels can be
// reported against measured as well as published peaks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla_probe.h"
#include "mla_host.h"

namespace mla_probe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kReadBlocksPerCu = 8;
constexpr int kMfmaBlocksPerCu = 2;      // 2 x 4 waves: two waves per SIMD
constexpr int kThreads = 256;
constexpr int kUnroll = 8;               // loads in flight per lane

// every lane reads 16 bytes per load, kUnroll loads in flight, grid-stride over the buffer
__global__ __launch_bounds__(kThreads) void hbm_read_kernel(const u32x4_t* __restrict__ src, size_t n16,
                                                            u32x4_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) v[k] = __builtin_nontemporal_load(src + i + k * stride);
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) acc ^= v[k];
  }
  for (; i < n16; i += stride) acc ^= src[i];
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

// four independent accumulation chains of 32x32x16 bf16 MFMAs per wave
__global__ __launch_bounds__(kThreads) void mfma_loop_kernel(float* __restrict__ sink, int iters) {
  const int t = threadIdx.x;
  bf16x8_t a, b;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = (__bf16)((float)((t + k) & 7) * 0.125f);
    b[k] = (__bf16)((float)((t * 3 + k) & 7) * 0.0625f);
  }
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) s += c0[k] + c1[k] + c2[k] + c3[k];
  sink[(size_t)blockIdx.x * kThreads + t] = s;
}

inline int cu_count() {
  mla::DeviceInfo di;
  if (mla::device_info(&di) != MLA_OK) return 0;
  return di.cu_count;
}

}  // namespace mla_probe

extern "C" size_t mla_probe_sink_bytes(void) {
  const int cus = mla_probe::cu_count();
  if (cus <= 0) return 0;
  const int blocks = cus * (mla_probe::kReadBlocksPerCu > mla_probe::kMfmaBlocksPerCu ? mla_probe::kReadBlocksPerCu
                                                                                       : mla_probe::kMfmaBlocksPerCu);
  return (size_t)blocks * mla_probe::kThreads * 16;
}

extern "C" double mla_probe_mfma_flops(int32_t iters) {
  const int cus = mla_probe::cu_count();
  return (double)cus * mla_probe::kMfmaBlocksPerCu * (mla_probe::kThreads / 64) * (double)iters * 4.0 * 32.0 *
         32.0 * 16.0 * 2.0;
}

extern "C" mla_status_t mla_probe_hbm_read(const void* src, size_t bytes, void* sink, void* stream) {
  if (!src || !sink) return MLA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(src) & 15u) || (reinterpret_cast<uintptr_t>(sink) & 15u) || (bytes & 15u))
    return MLA_ERR_ALIGN;
  mla::DeviceInfo di;
  const mla_status_t st = mla::device_info(&di);
  if (st != MLA_OK) return st;
  const dim3 grid((unsigned)(di.cu_count * mla_probe::kReadBlocksPerCu));
  hipLaunchKernelGGL(mla_probe::hbm_read_kernel, grid, dim3(mla_probe::kThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const mla_probe::u32x4_t*>(src), bytes / 16,
                     static_cast<mla_probe::u32x4_t*>(sink));
  return mla::launch_status();
}

extern "C" mla_status_t mla_probe_mfma_bf16(float* sink, int32_t iters, void* stream) {
  if (!sink) return MLA_ERR_NULL;
  if (iters < 1 || iters > (1 << 24)) return MLA_ERR_SHAPE;
  mla::DeviceInfo di;
  const mla_status_t st = mla::device_info(&di);
  if (st != MLA_OK) return st;
  const dim3 grid((unsigned)(di.cu_count * mla_probe::kMfmaBlocksPerCu));
  hipLaunchKernelGGL(mla_probe::mfma_loop_kernel, grid, dim3(mla_probe::kThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), sink, iters);
  return mla::launch_status();
}
