// KDA chunked prefill (export kda_chunk_prefill) -- placeholder until the
// chunk kernels land.
#include "kda_device.h"
#include "kda_host.h"

extern "C" int kda_chunk_prefill(const void*, const void*, const void*, const float*, const void*,
                                 const float*, const int32_t*, int32_t, int32_t, int32_t,
                                 int32_t, int32_t, int32_t, int32_t, void*, float*, void*) {
  return KDA_ERR_UNSUPPORTED;
}
