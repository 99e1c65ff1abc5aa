// Host-side helpers shared by the entry points: status handling and
// metadata checks.  No allocation, no synchronisation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/kda.h"

namespace kda {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Compute units of the current device, cached per device (256, MI355X's
// count, when the runtime reports no device).  Launch shapes and the choice
// between kernels follow it.
inline int device_cus() {
  constexpr int kDevices = 64;
  static std::atomic<int> cache[kDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevices) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

// Map the runtime's view of the most recent launch to a status.
inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace kda
