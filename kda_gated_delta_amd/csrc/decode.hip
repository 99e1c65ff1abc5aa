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
// then LDS across the four waves; everything is float32.  Small batches run
// a second kernel with the same arithmetic in finer pieces (see
// decode_quarter_kernel below).
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
  // The decay of channel j: loaded (decay_load), then formed (decay_of).
  struct DecayIn {
    float g;
  };
  __device__ DecayIn decay_load(int b, int hv, int HV, int j) const { return {g[(int64_t(b) * HV + hv) * K + j]}; }
  __device__ float decay_of(const DecayIn& d) const { return expf(d.g); }
  __device__ uint16_t value_load(int b, int hv, int HV, int j) const { return v[(int64_t(b) * HV + hv) * V + j]; }
  __device__ uint4 value8(int b, int hv, int HV, int j0) const {
    return *reinterpret_cast<const uint4*>(v + (int64_t(b) * HV + hv) * V + j0);
  }
  __device__ uint16_t beta_load(int b, int hv, int HV) const { return beta[int64_t(b) * HV + hv]; }
  __device__ float beta_of(uint16_t raw) const { return kda::bf16f(raw); }
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
  struct DecayIn {
    uint16_t raw;
    float bias, alog;
  };
  __device__ DecayIn decay_load(int b, int hv, int HV, int j) const {
    return {raw_gate[(int64_t(b) * HV + hv) * K + j], dt_bias[hv * K + j], A_log[hv]};
  }
  __device__ float decay_of(const DecayIn& d) const {
    const float x = kda::bf16f(d.raw) + d.bias;
    const float z = expf(d.alog) * x;
    return expf(kLowerBound / (1.0f + expf(-z)));
  }
  __device__ uint16_t value_load(int b, int hv, int HV, int j) const {
    return qkv[int64_t(b) * row_stride + 2 * HV * K + hv * V + j];
  }
  __device__ uint4 value8(int b, int hv, int HV, int j0) const {
    return *reinterpret_cast<const uint4*>(qkv + int64_t(b) * row_stride + 2 * HV * K + hv * V + j0);
  }
  __device__ uint16_t beta_load(int b, int hv, int HV) const { return raw_beta[int64_t(b) * HV + hv]; }
  __device__ float beta_of(uint16_t raw) const { return 1.0f / (1.0f + expf(-kda::bf16f(raw))); }
};

// An empty asm that claims to change its operand: nothing that reads the
// value can move above it, and the load that produced it must be complete
// there.  Used to hold a wave's per-row inputs until its state loads are
// issued.
__device__ __forceinline__ void pin(uint32_t& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(uint16_t& x) {
  uint32_t y = x;
  pin(y);
  x = uint16_t(y);
}
__device__ __forceinline__ void pin(float& x) {
  uint32_t y = __builtin_bit_cast(uint32_t, x);
  pin(y);
  x = __builtin_bit_cast(float, y);
}
__device__ __forceinline__ void pin(uint4& x) {
  pin(x.x);
  pin(x.y);
  pin(x.z);
  pin(x.w);
}
__device__ __forceinline__ void pin(SplitInputs::DecayIn& d) { pin(d.g); }
__device__ __forceinline__ void pin(PackedInputs::DecayIn& d) {
  pin(d.raw);
  pin(d.bias);
  pin(d.alog);
}

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

  // The per-row inputs are loaded before the state: the vector-memory counter
  // completes in order, so waiting for them leaves the 32 KB of state in
  // flight while the norm and the decay are formed (measured 3% faster, and
  // 8% for the packed inputs, whose decay takes three exponentials).  Every
  // wave issues all of them at the same addresses (the copies hit in the
  // caches) and pins them after its state loads, so that neither the loads
  // nor their uses move into the per-wave branches, where a masked-off path
  // would wait for them.
  const int l64 = t & 63;
  uint4 xl = *(in.qk_row(b, hv, HV, l64 >= 16) + (l64 & 15));   // lanes 0-15 q, 16-31 k
  typename In::DecayIn d0 = in.decay_load(b, hv, HV, l64);
  typename In::DecayIn d1 = in.decay_load(b, hv, HV, l64 + 64);
  uint16_t vr0 = in.value_load(b, hv, HV, l64);
  uint16_t vr1 = in.value_load(b, hv, HV, l64 + 64);
  const uint16_t braw = in.beta_load(b, hv, HV);

  uint4* slot = reinterpret_cast<uint4*>(pool + idx * slot_stride + int64_t(hv) * K * V);
  uint4 sv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sv[i] = slot[(kr + 16 * i) * (V / 8) + cg];
  pin(xl);
  pin(d0);
  pin(d1);
  pin(vr0);
  pin(vr1);

  if (wave == 0) {
    const int lane = t;
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
    s_eg[l64] = in.decay_of(d0);
    s_eg[l64 + 64] = in.decay_of(d1);
  } else if (wave == 2) {
    s_v[l64] = kda::bf16f(vr0);
    s_v[l64 + 64] = kda::bf16f(vr1);
  }
  const float bt = in.beta_of(braw);
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
  // S' = S_decay + beta k r^T, stored rounded to bf16 in place, with the
  // nontemporal hint (the slot is not read again by this step; measured 2.5%
  // faster at B = 256 after a prefill, where the same hint on the loads was
  // slower).
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float bk = bt * s_k[kr + 16 * i];
    uint4 out;
    out.x = kda::pack_bf16(fmaf(bk, rr[0], sd[i][0]), fmaf(bk, rr[1], sd[i][1]));
    out.y = kda::pack_bf16(fmaf(bk, rr[2], sd[i][2]), fmaf(bk, rr[3], sd[i][3]));
    out.z = kda::pack_bf16(fmaf(bk, rr[4], sd[i][4]), fmaf(bk, rr[5], sd[i][5]));
    out.w = kda::pack_bf16(fmaf(bk, rr[6], sd[i][6]), fmaf(bk, rr[7], sd[i][7]));
    kda::store_nt(&slot[(kr + 16 * i) * (V / 8) + cg], out);
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

// ---------------------------------------------------------------------------
// Small batches.  With few (row, value head) pairs the grid above leaves
// most compute units idle, so each pair is split four ways by state columns
// -- the page's operator likewise picks a narrower value tile for small
// batches.  Column c of S' needs only column c of S, v_c and the shared q,
// k, g and beta, so the quarters are independent: one single-wave
// workgroup per quarter, which normalises q and k itself and streams its
// 128x32 slice (8 KB in, 8 KB out).  Lane l owns columns
// 32 * quarter + 8 (l % 4) .. +7 of rows l / 4 + 16 i, i < 8.
//
// Measured on MI355X (HV = 12, a cold cache): 7.6 against 8.4 us at B = 1
// and 8.3 against 8.6 us at B = 4, where the quarters still take one
// compute unit each; from B = 8 (384 quarters on 256 compute units) the
// row kernel is faster (8.8 against 9.4 us, 37 against 53 us at B = 256).
// So the quarters run while 4 B HV is at most the number of compute units.
//
// The arithmetic and its order are those of decode_kernel, so both kernels
// give the same bits and a row's result does not depend on the batch it is
// decoded in.  In particular lane l's rows are those of decode_kernel's
// thread with row group l / 4, and the column sums combine the per-lane
// partial sums over lane bits 2-3 and then 4-5 as butterflies, which forms
// (p0 + p1) + (p2 + p3) within each group of four row groups and then
// (W0 + W1) + (W2 + W3) over the groups -- what decode_kernel's two shuffles
// and its cross-wave sum form.
template <int XOR>
__device__ __forceinline__ float swizzle_xor(float x) {
  // ds_swizzle bit-mask mode within 32 lanes: source lane = lane ^ XOR.
  static_assert(XOR > 0 && XOR < 32, "swizzle reaches within 32 lanes");
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x1f | (XOR << 10)));
}

__device__ __forceinline__ float colgroup_sum(float x) {
  x += swizzle_xor<4>(x);
  x += swizzle_xor<8>(x);
  x += swizzle_xor<16>(x);
  x += __shfl_xor(x, 32, 64);
  return x;
}

template <class In>
__global__ __launch_bounds__(64) void decode_quarter_kernel(In in, uint16_t* __restrict__ pool,
                                                            int64_t slot_stride, int64_t num_slots,
                                                            const int32_t* __restrict__ state_indices, int HV,
                                                            uint4* __restrict__ o) {
  __shared__ float s_x[3][K];   // q^, k^, exp(g)

  const int lane = threadIdx.x;
  const int hv = blockIdx.x >> 2;
  const int b = blockIdx.y;
  const int rg = lane >> 2;                                // rows rg + 16 i
  const int c0 = 32 * (blockIdx.x & 3) + 8 * (lane & 3);   // columns c0 .. c0 + 7
  const int64_t row_head = int64_t(b) * HV + hv;

  const int64_t idx = state_indices[b];
  if (idx < 0 || idx >= num_slots) {   // inactive row: zero output, no pool access
    if (rg == 0) o[row_head * (V / 8) + c0 / 8] = make_uint4(0u, 0u, 0u, 0u);
    return;
  }

  // Per-row inputs first, then the state, as in decode_kernel.  q^ (lanes
  // 0-15) and k^ (lanes 16-31), 8 elements per lane; lanes 32-63 normalise a
  // zero row alongside.
  uint4 xl = *(in.qk_row(b, hv, HV, (lane & 16) != 0) + (lane & 15));
  uint4 vv = in.value8(b, hv, HV, c0);
  typename In::DecayIn d0 = in.decay_load(b, hv, HV, lane);
  typename In::DecayIn d1 = in.decay_load(b, hv, HV, lane + 64);
  const uint16_t braw = in.beta_load(b, hv, HV);

  uint4* slot = reinterpret_cast<uint4*>(pool + idx * slot_stride + int64_t(hv) * K * V);
  uint4 sv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sv[i] = slot[((rg + 16 * i) * V + c0) / 8];
  pin(xl);
  pin(vv);
  pin(d0);
  pin(d1);

  const uint4 x = lane < 32 ? xl : make_uint4(0u, 0u, 0u, 0u);
  const float e0 = in.decay_of(d0), e1 = in.decay_of(d1);
  const float bt = in.beta_of(braw);
  const uint4 y = kda::l2norm_row16(x);
  if (lane < 32) {
    float* dst = s_x[lane < 16 ? 0 : 1] + (lane & 15) * 8;
    const uint32_t w[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      dst[2 * p] = kda::bf16lo(w[p]);
      dst[2 * p + 1] = kda::bf16hi(w[p]);
    }
  }
  s_x[2][lane] = e0;
  s_x[2][lane + 64] = e1;
  __syncthreads();   // a one-wave workgroup

  // The decayed state's column sums against k^ and q^, and q^.k^.
  float pk[8], pq[8], pqk = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) pk[j] = pq[j] = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = rg + 16 * i;
    const float e = s_x[2][r], kk = s_x[1][r], qq = s_x[0][r];
    const uint32_t w[4] = {sv[i].x, sv[i].y, sv[i].z, sv[i].w};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float d0 = e * kda::bf16lo(w[p]), d1 = e * kda::bf16hi(w[p]);
      pk[2 * p] = fmaf(kk, d0, pk[2 * p]);
      pk[2 * p + 1] = fmaf(kk, d1, pk[2 * p + 1]);
      pq[2 * p] = fmaf(qq, d0, pq[2 * p]);
      pq[2 * p + 1] = fmaf(qq, d1, pq[2 * p + 1]);
    }
    pqk = fmaf(qq, kk, pqk);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    pk[j] = colgroup_sum(pk[j]);
    pq[j] = colgroup_sum(pq[j]);
  }
  pqk = colgroup_sum(pqk);

  // S' = exp(g) S + beta k^ r^T with r = v - k^T (exp(g) S), stored rounded
  // to bf16 in place (the decayed entries recomputed exactly as above).
  const uint32_t vw[4] = {vv.x, vv.y, vv.z, vv.w};
  float rr[8];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    rr[2 * p] = kda::bf16lo(vw[p]) - pk[2 * p];
    rr[2 * p + 1] = kda::bf16hi(vw[p]) - pk[2 * p + 1];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = rg + 16 * i;
    const float e = s_x[2][r], bk = bt * s_x[1][r];
    const uint32_t w[4] = {sv[i].x, sv[i].y, sv[i].z, sv[i].w};
    uint32_t out[4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
      out[p] = kda::pack_bf16(fmaf(bk, rr[2 * p], e * kda::bf16lo(w[p])),
                              fmaf(bk, rr[2 * p + 1], e * kda::bf16hi(w[p])));
    slot[(r * V + c0) / 8] = make_uint4(out[0], out[1], out[2], out[3]);
  }
  // o = K^-1/2 (q^T exp(g) S + beta (q^.k^) r), from the unrounded S'.
  if (rg == 0) {
    const float scale = 0.08838834764831845f;   // 128^-1/2
    float ov[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) ov[j] = scale * fmaf(bt * pqk, rr[j], pq[j]);
    o[row_head * (V / 8) + c0 / 8] = make_uint4(kda::pack_bf16(ov[0], ov[1]), kda::pack_bf16(ov[2], ov[3]),
                                               kda::pack_bf16(ov[4], ov[5]), kda::pack_bf16(ov[6], ov[7]));
  }
}

// Both kernels, chosen by the number of (row, value head) pairs.
template <class In>
int launch_decode(const In& in, uint16_t* pool, int64_t slot_stride, int64_t num_slots,
                  const int32_t* state_indices, int B, int HV, uint4* o, hipStream_t stream) {
  if (int64_t(4) * B * HV <= kda::device_cus())
    hipLaunchKernelGGL(decode_quarter_kernel<In>, dim3(4 * HV, B), dim3(64), 0, stream, in, pool, slot_stride,
                       num_slots, state_indices, HV, o);
  else
    hipLaunchKernelGGL(decode_kernel<In>, dim3(HV, B), dim3(256), 0, stream, in, pool, slot_stride, num_slots,
                       state_indices, HV, o);
  return kda::launch_status();
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
  if (!kda::aligned16(q) || !kda::aligned16(k) || !kda::aligned16(v) || !kda::aligned16(o) ||
      (state_pool && !kda::aligned16(state_pool)))
    return KDA_ERR_ALIGN;
  if (B > 65535 || HV > (1 << 28)) return KDA_ERR_SHAPE;
  SplitInputs in;
  in.q = static_cast<const uint4*>(q);
  in.k = static_cast<const uint4*>(k);
  in.v = static_cast<const uint16_t*>(v);
  in.g = g;
  in.beta = static_cast<const uint16_t*>(beta);
  in.H = H;
  return launch_decode(in, static_cast<uint16_t*>(state_pool), slot_stride, num_slots, state_indices, B, HV,
                       static_cast<uint4*>(o), kda::as_stream(stream));
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
  if (B > 65535 || H > (1 << 28)) return KDA_ERR_SHAPE;
  PackedInputs in;
  in.qkv = static_cast<const uint16_t*>(mixed_qkv);
  in.row_stride = qkv_row_stride;
  in.raw_gate = static_cast<const uint16_t*>(raw_gate);
  in.raw_beta = static_cast<const uint16_t*>(raw_beta);
  in.A_log = A_log;
  in.dt_bias = dt_bias;
  return launch_decode(in, static_cast<uint16_t*>(state_pool), slot_stride, num_slots, state_indices, B, H,
                       static_cast<uint4*>(o), kda::as_stream(stream));
}
