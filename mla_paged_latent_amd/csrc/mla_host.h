// Host-side helpers shared by the C-ABI entry points: device capability cache,
// argument checks and launch error mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cstring>

#include "../../include/mla.h"

namespace mla {

struct DeviceInfo {
  int cu_count = 0;
  bool gfx950 = false;
};

// Per-device properties, read once per device and cached (benign race: every
// writer stores the same values).
inline mla_status_t device_info(DeviceInfo* info) {
  constexpr int kMaxDev = 64;
  static std::atomic<int> state[kMaxDev];        // 0 = unknown, 1 = filled
  static DeviceInfo cache[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return MLA_ERR_HIP;
  if (state[dev].load(std::memory_order_acquire) == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MLA_ERR_HIP;
    DeviceInfo d;
    d.cu_count = prop.multiProcessorCount;
    d.gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    cache[dev] = d;
    state[dev].store(1, std::memory_order_release);
  }
  *info = cache[dev];
  return info->gfx950 ? MLA_OK : MLA_ERR_DEVICE;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool mult8(int64_t s) { return (s & 7) == 0; }

inline mla_status_t launch_status() {
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // namespace mla
