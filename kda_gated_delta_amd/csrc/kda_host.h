// Host-side helpers shared by the entry points: status handling and
// metadata checks.  No allocation, no synchronisation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kda.h"

namespace kda {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Map the runtime's view of the most recent launch to a status.
inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace kda
