// Standalone bit-exact Q/K row normalisation (the export kda_qk_l2norm).
//
// Page "KDA Chunk Prefill on Ascend A3", section "Mathematical definition".
// One 16-lane group per row, 8 bf16 per lane (one 16-byte load and store);
// a 256-thread workgroup normalises 16 rows.
#include "kda_device.h"
#include "kda_host.h"

namespace {

constexpr int kRowsPerBlock = 16;

__global__ __launch_bounds__(256) void qk_l2norm_kernel(const uint4* __restrict__ x,
                                                         uint4* __restrict__ y,
                                                         int64_t rows) {
  const int lane16 = threadIdx.x & 15;
  const int64_t row = int64_t(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 4);
  const bool valid = row < rows;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (valid) v = x[row * 16 + lane16];
  uint4 r = kda::l2norm_row16(v);   // every lane takes part in the shuffles
  if (valid) y[row * 16 + lane16] = r;
}

}  // namespace

extern "C" int kda_qk_l2norm(const void* x, void* y, int64_t rows, int32_t K, void* stream) {
  if (rows < 0) return KDA_ERR_SHAPE;
  if (K != kda::kHead) return KDA_ERR_UNSUPPORTED;
  if (rows == 0) return KDA_OK;
  if (!x || !y) return KDA_ERR_NULL;
  if (!kda::aligned16(x) || !kda::aligned16(y)) return KDA_ERR_ALIGN;
  const int64_t blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (blocks > 0x7fffffff) return KDA_ERR_SHAPE;
  hipLaunchKernelGGL(qk_l2norm_kernel, dim3(unsigned(blocks)), dim3(256), 0, kda::as_stream(stream),
                     static_cast<const uint4*>(x), static_cast<uint4*>(y), rows);
  return kda::launch_status();
}
