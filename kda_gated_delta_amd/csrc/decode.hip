// Single-token KDA decode against a bf16 state pool (exports kda_decode and,
// from the page's packed serving inputs, kda_packed_decode).
//
// Pages: "flashinfer.kda_decode.packed_kda_decode" (section "Parameters":
// bf16 pool [N, HV, K, V] updated in place, -1 rows inactive) and "KDA Chunk
// Prefill on Ascend A3" (section "Mathematical definition": the recurrent
// step and the Q/K normalisation).
//
// One 256-thread workgroup per (row, value head) streams that slot's
// 128x128 bf16 state once in and once out (32 KB each way), which is all
// but ~1% of the bytes: the kernel is HBM-bound.  Thread t owns columns
// 8*(t%16) .. +7 of rows (t/16) + 16*i, i < 8, so every 16-byte load and
// store is coalesced (a wave covers four whole 256-byte rows).  The two
// column reductions over K (k^T S and q^T S) go through lane shuffles and
// then LDS across the four waves; everything is float32.
#include "kda_device.h"
#include "kda_host.h"

namespace {

constexpr int K = kda::kHead;
constexpr int V = kda::kHead;

// Where one decode step reads its per-row inputs.  The kernel is the same
// for both forms; only these accessors differ.

// Separate tensors: q, k [B, H, K]; v [B, HV, V]; g [B, HV, K] (log decay);
// beta [B, HV].  Value head hv reads Q/K head hv / (HV / H).
struct SplitInputs {
  const uint4* q;
  const uint4* k;
  const uint16_t* v;
  const float* g;
  const uint16_t* beta;
  int H;
  __device__ const uint4* qk_row(int b, int hv, int HV, bool key) const {
    const int hq = hv / (HV / H);
    return (key ? k : q) + (int64_t(b) * H + hq) * (K / 8);
  }
  __device__ float decay(int b, int hv, int HV, int j) const {
    return expf(g[(int64_t(b) * HV + hv) * K + j]);
  }
  __device__ float value(int b, int hv, int HV, int j) const {
    return kda::bf16f(v[(int64_t(b) * HV + hv) * V + j]);
  }
  __device__ float beta_of(int b, int hv, int HV) const { return kda::bf16f(beta[int64_t(b) * HV + hv]); }
};

// Page "flashinfer.kda_decode.packed_kda_decode": one packed bf16 row per
// batch row holding q | k | v (each [H, 128], head-major; H == HV), raw
// gate logits [B, H*K], raw beta logits [B, H], per-head A_log and
// per-channel dt_bias.  The lower-bound gate transform (lower_bound = -5)
// is read as g = -5 * sigmoid(exp(A_log[h]) * (raw + dt_bias)) -- the page
// names the transform and its parameters but not the formula -- and
// beta = sigmoid(raw_beta).  All in float32.
struct PackedInputs {
  const uint16_t* qkv;
  int64_t row_stride;
  const uint16_t* raw_gate;
  const uint16_t* raw_beta;
  const float* A_log;
  const float* dt_bias;
  static constexpr float kLowerBound = -5.0f;
  __device__ const uint4* qk_row(int b, int hv, int HV, bool key) const {
    return reinterpret_cast<const uint4*>(qkv + int64_t(b) * row_stride + (key ? HV * K : 0) + hv * K);
  }
  __device__ float decay(int b, int hv, int HV, int j) const {
    const float x = kda::bf16f(raw_gate[(int64_t(b) * HV + hv) * K + j]) + dt_bias[hv * K + j];
    const float z = expf(A_log[hv]) * x;
    return expf(kLowerBound / (1.0f + expf(-z)));
  }
  __device__ float value(int b, int hv, int HV, int j) const {
    return kda::bf16f(qkv[int64_t(b) * row_stride + 2 * HV * K + hv * V + j]);
  }
  __device__ float beta_of(int b, int hv, int HV) const {
    return 1.0f / (1.0f + expf(-kda::bf16f(raw_beta[int64_t(b) * HV + hv])));
  }
};

template <class In>
__global__ __launch_bounds__(256) void decode_kernel(In in, uint16_t* __restrict__ pool, int64_t slot_stride,
                                                     int64_t num_slots, const int32_t* __restrict__ state_indices,
                                                     int HV, uint4* __restrict__ o) {
  __shared__ float s_q[K], s_k[K], s_eg[K], s_v[V];
  __shared__ float s_red[3][4][V];   // [k^T S | q^T S | q.k][wave][column]

  const int t = threadIdx.x;
  const int hv = blockIdx.x;
  const int b = blockIdx.y;
  const int cg = t & 15;        // column group: columns 8*cg .. 8*cg+7
  const int kr = t >> 4;        // row group: rows kr + 16*i
  const int wave = t >> 6;
  const int64_t row_head = int64_t(b) * HV + hv;

  const int64_t idx = state_indices[b];
  if (idx < 0 || idx >= num_slots) {   // inactive row: zero output, no pool access
    if (t < 16) o[row_head * (V / 8) + t] = make_uint4(0u, 0u, 0u, 0u);
    return;
  }

  uint4* slot = reinterpret_cast<uint4*>(pool + idx * slot_stride + int64_t(hv) * K * V);
  uint4 sv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sv[i] = slot[(kr + 16 * i) * (V / 8) + cg];

  if (wave == 0) {
    // Lanes 0-15 hold the q row, 16-31 the k row; the loads are unconditional
    // (a load inside a branch would be waited for inside it).
    const int lane = t;
    const uint4* src = in.qk_row(b, hv, HV, lane >= 16) + (lane & 15);
    const uint4 xl = *src;
    const uint4 x = lane < 32 ? xl : make_uint4(0u, 0u, 0u, 0u);
    uint4 y = kda::l2norm_row16(x);
    float* dst = lane < 16 ? s_q : s_k;
    if (lane < 32) {
      const int c0 = (lane & 15) * 8;
      const uint32_t w[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dst[c0 + 2 * i] = kda::bf16lo(w[i]);
        dst[c0 + 2 * i + 1] = kda::bf16hi(w[i]);
      }
    }
  } else if (wave == 1) {
    const int j = t - 64;
    s_eg[j] = in.decay(b, hv, HV, j);
    s_eg[j + 64] = in.decay(b, hv, HV, j + 64);
  } else if (wave == 2) {
    const int j = t - 128;
    s_v[j] = in.value(b, hv, HV, j);
    s_v[j + 64] = in.value(b, hv, HV, j + 64);
  }
  const float bt = in.beta_of(b, hv, HV);
  __syncthreads();

  float sd[8][8];
  float pk[8], pq[8], pqk = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) pk[j] = pq[j] = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = kr + 16 * i;
    const float e = s_eg[r], kk = s_k[r], qq = s_q[r];
    const uint32_t w[4] = {sv[i].x, sv[i].y, sv[i].z, sv[i].w};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      sd[i][2 * p] = e * kda::bf16lo(w[p]);
      sd[i][2 * p + 1] = e * kda::bf16hi(w[p]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pk[j] = fmaf(kk, sd[i][j], pk[j]);
      pq[j] = fmaf(qq, sd[i][j], pq[j]);
    }
    pqk = fmaf(qq, kk, pqk);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    pk[j] += __shfl_xor(pk[j], 16, 64);
    pk[j] += __shfl_xor(pk[j], 32, 64);
    pq[j] += __shfl_xor(pq[j], 16, 64);
    pq[j] += __shfl_xor(pq[j], 32, 64);
  }
  pqk += __shfl_xor(pqk, 16, 64);
  pqk += __shfl_xor(pqk, 32, 64);
  if ((t & 63) < 16) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      s_red[0][wave][cg * 8 + j] = pk[j];
      s_red[1][wave][cg * 8 + j] = pq[j];
    }
    if (cg == 0) s_red[2][wave][0] = pqk;
  }
  __syncthreads();

  float rr[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = cg * 8 + j;
    const float kd = (s_red[0][0][c] + s_red[0][1][c]) + (s_red[0][2][c] + s_red[0][3][c]);
    rr[j] = s_v[c] - kd;
  }
  // S' = S_decay + beta k r^T, stored rounded to bf16 in place.
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float bk = bt * s_k[kr + 16 * i];
    uint4 out;
    out.x = kda::pack_bf16(fmaf(bk, rr[0], sd[i][0]), fmaf(bk, rr[1], sd[i][1]));
    out.y = kda::pack_bf16(fmaf(bk, rr[2], sd[i][2]), fmaf(bk, rr[3], sd[i][3]));
    out.z = kda::pack_bf16(fmaf(bk, rr[4], sd[i][4]), fmaf(bk, rr[5], sd[i][5]));
    out.w = kda::pack_bf16(fmaf(bk, rr[6], sd[i][6]), fmaf(bk, rr[7], sd[i][7]));
    slot[(kr + 16 * i) * (V / 8) + cg] = out;
  }
  // o = K^-1/2 q^T S' = K^-1/2 (q^T S_decay + beta (q.k) r), from the unrounded S'.
  if (kr == 0) {
    const float qk = (s_red[2][0][0] + s_red[2][1][0]) + (s_red[2][2][0] + s_red[2][3][0]);
    const float scale = 0.08838834764831845f;   // 128^-1/2
    float ov[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = cg * 8 + j;
      const float qd = (s_red[1][0][c] + s_red[1][1][c]) + (s_red[1][2][c] + s_red[1][3][c]);
      ov[j] = scale * fmaf(bt * qk, rr[j], qd);
    }
    uint4 out;
    out.x = kda::pack_bf16(ov[0], ov[1]);
    out.y = kda::pack_bf16(ov[2], ov[3]);
    out.z = kda::pack_bf16(ov[4], ov[5]);
    out.w = kda::pack_bf16(ov[6], ov[7]);
    o[row_head * (V / 8) + cg] = out;
  }
}

}  // namespace

extern "C" int kda_decode(const void* q, const void* k, const void* v, const float* g,
                          const void* beta, void* state_pool, int64_t slot_stride,
                          int64_t num_slots, const int32_t* state_indices, int32_t B,
                          int32_t H, int32_t HV, int32_t Kd, int32_t Vd, void* o,
                          void* stream) {
  if (B < 0 || H < 1 || HV < 1 || HV % H != 0 || num_slots < 0) return KDA_ERR_SHAPE;
  if (Kd != K || Vd != V) return KDA_ERR_UNSUPPORTED;
  if (B == 0) return KDA_OK;
  if (!q || !k || !v || !g || !beta || !state_indices || !o) return KDA_ERR_NULL;
  if (num_slots > 0 && !state_pool) return KDA_ERR_NULL;
  if (slot_stride < int64_t(HV) * K * V) return KDA_ERR_SHAPE;
  if (slot_stride % 8 != 0) return KDA_ERR_ALIGN;
  if (!kda::aligned16(q) || !kda::aligned16(k) || !kda::aligned16(o) ||
      (state_pool && !kda::aligned16(state_pool)))
    return KDA_ERR_ALIGN;
  if (B > 65535) return KDA_ERR_SHAPE;
  SplitInputs in;
  in.q = static_cast<const uint4*>(q);
  in.k = static_cast<const uint4*>(k);
  in.v = static_cast<const uint16_t*>(v);
  in.g = g;
  in.beta = static_cast<const uint16_t*>(beta);
  in.H = H;
  hipLaunchKernelGGL(decode_kernel<SplitInputs>, dim3(HV, B), dim3(256), 0, kda::as_stream(stream), in,
                     static_cast<uint16_t*>(state_pool), slot_stride, num_slots, state_indices, int(HV),
                     static_cast<uint4*>(o));
  return kda::launch_status();
}

extern "C" int kda_packed_decode(const void* mixed_qkv, int64_t qkv_row_stride, const void* raw_gate,
                                 const void* raw_beta, const float* A_log, const float* dt_bias,
                                 void* state_pool, int64_t slot_stride, int64_t num_slots,
                                 const int32_t* state_indices, int32_t B, int32_t H, int32_t Kd,
                                 int32_t Vd, void* o, void* stream) {
  if (B < 0 || H < 1 || num_slots < 0) return KDA_ERR_SHAPE;
  if (Kd != K || Vd != V) return KDA_ERR_UNSUPPORTED;
  if (B == 0) return KDA_OK;
  if (!mixed_qkv || !raw_gate || !raw_beta || !A_log || !dt_bias || !state_indices || !o)
    return KDA_ERR_NULL;
  if (num_slots > 0 && !state_pool) return KDA_ERR_NULL;
  if (qkv_row_stride < int64_t(3) * H * K) return KDA_ERR_SHAPE;
  if (slot_stride < int64_t(H) * K * V) return KDA_ERR_SHAPE;
  if (qkv_row_stride % 8 != 0 || slot_stride % 8 != 0) return KDA_ERR_ALIGN;
  if (!kda::aligned16(mixed_qkv) || !kda::aligned16(o) || (state_pool && !kda::aligned16(state_pool)))
    return KDA_ERR_ALIGN;
  if (B > 65535) return KDA_ERR_SHAPE;
  PackedInputs in;
  in.qkv = static_cast<const uint16_t*>(mixed_qkv);
  in.row_stride = qkv_row_stride;
  in.raw_gate = static_cast<const uint16_t*>(raw_gate);
  in.raw_beta = static_cast<const uint16_t*>(raw_beta);
  in.A_log = A_log;
  in.dt_bias = dt_bias;
  hipLaunchKernelGGL(decode_kernel<PackedInputs>, dim3(H, B), dim3(256), 0, kda::as_stream(stream), in,
                     static_cast<uint16_t*>(state_pool), slot_stride, num_slots, state_indices, int(H),
                     static_cast<uint4*>(o));
  return kda::launch_status();
}
