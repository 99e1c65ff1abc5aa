// Prefill-to-decode handoff (export kda_state_to_pool): the float32 final
// states of a prefill stored, rounded once to bfloat16, into the decode
// state pool.
//
// Pages: "KDA Chunk Prefill on Ascend A3" (section "Function and tensor
// contract": the prefill returns an fp32 final state per sequence and value
// head) and "flashinfer.kda_decode.packed_kda_decode" (section "Parameters":
// the decode keeps its recurrent state in a caller-owned bf16 pool
// [N, HV, K, V] with compact inner dimensions, a free slot stride and int32
// slot indices where -1 means no state access).
//
// Pure streaming: per (sequence, value head) 64 KB of fp32 in and 32 KB of
// bf16 out.  A 256-thread workgroup converts one eighth of a state (2048
// elements): each thread issues both of its 16-byte loads before its store
// of eight bf16.  A wave covers whole 256-byte pool rows, so every access is
// coalesced.  (Eighths measured faster than quarters or halves of a state
// per workgroup; the nontemporal hint measured slower after a prefill.)
#include "kda_device.h"
#include "kda_host.h"

namespace {

constexpr int K = kda::kHead;
constexpr int V = kda::kHead;
constexpr int kParts = 8;                       // workgroups per state
constexpr int kPerBlock = K * V / kParts;       // 2048 elements
constexpr int kThreads = 256;
static_assert(kPerBlock == 8 * kThreads, "one group of eight elements per thread");

__global__ __launch_bounds__(kThreads) void state_to_pool_kernel(
    const float4* __restrict__ state, uint16_t* __restrict__ pool, int64_t slot_stride,
    int64_t num_slots, const int32_t* __restrict__ state_indices, int HV) {
  const int64_t sh = blockIdx.x / kParts;       // state (sequence n, head hv), row-major
  const int part = blockIdx.x - sh * kParts;
  const int n = int(sh / HV);
  const int hv = int(sh - int64_t(n) * HV);
  const int64_t idx = state_indices[n];
  if (idx < 0 || idx >= num_slots) return;      // no pool access for this sequence

  const float4* src = state + sh * (K * V / 4) + part * (kPerBlock / 4);
  uint4* dst = reinterpret_cast<uint4*>(pool + idx * slot_stride + int64_t(hv) * K * V +
                                        part * kPerBlock);
  const int t = threadIdx.x;
  // Thread t converts elements 8t..8t+7 of the part.
  const float4 a = src[2 * t];
  const float4 b = src[2 * t + 1];
  dst[t] = make_uint4(kda::pack_bf16(a.x, a.y), kda::pack_bf16(a.z, a.w), kda::pack_bf16(b.x, b.y),
                      kda::pack_bf16(b.z, b.w));
}

}  // namespace

extern "C" int kda_state_to_pool(const float* state, int32_t N, int32_t HV, int32_t Kd, int32_t Vd,
                                 void* state_pool, int64_t slot_stride, int64_t num_slots,
                                 const int32_t* state_indices, void* stream) {
  if (N < 0 || HV < 1 || num_slots < 0) return KDA_ERR_SHAPE;
  if (Kd != K || Vd != V) return KDA_ERR_UNSUPPORTED;
  if (N == 0) return KDA_OK;
  if (!state || !state_indices) return KDA_ERR_NULL;
  if (num_slots > 0 && !state_pool) return KDA_ERR_NULL;
  if (slot_stride < int64_t(HV) * K * V) return KDA_ERR_SHAPE;
  if (slot_stride % 8 != 0) return KDA_ERR_ALIGN;
  if (!kda::aligned16(state) || (state_pool && !kda::aligned16(state_pool))) return KDA_ERR_ALIGN;
  const int64_t blocks = int64_t(N) * HV * kParts;
  if (blocks > 0x7fffffff) return KDA_ERR_SHAPE;
  hipLaunchKernelGGL(state_to_pool_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0,
                     kda::as_stream(stream), reinterpret_cast<const float4*>(state),
                     static_cast<uint16_t*>(state_pool), slot_stride, num_slots, state_indices,
                     int(HV));
  return kda::launch_status();
}
