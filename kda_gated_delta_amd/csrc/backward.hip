// KDA chunked backward (exports kda_chunk_backward and
// kda_chunk_backward_workspace_size).
//
// Page "KDA Chunk Prefill on Ascend A3": section "Function and tensor
// contract" (the optional backward: gradients of o and final_state with
// respect to q, k, v, g, beta and initial_state) and section "Mathematical
// definition" (the chunk construction whose gradients are taken: G, L,
// A = solve(I+L, diag(beta)), W, U, Qg, Kg, Aqk, the carry Vnew = U - W S,
// O = Qg S + Aqk Vnew, S' = exp(G_last) S + Kg^T Vnew, chunk size 64 with a
// zero-padded last chunk).  The page gives no backward formulas; these are
// the exact derivatives of that construction, which equals the token
// recurrence, so they are the recurrence's gradients.  The bf16 rounding of
// the normalised q and k passes gradients through unchanged: dq and dk are
// the gradients of x / sqrt(sum(x*x) + 1e-6).
//
// Everything runs in float32.  Five kernels, split where the method splits
// (chunk-local work is chunk-parallel, the carries are sequential per
// (sequence, value head) and column-parallel, since column v of the state
// only ever meets column v of the values):
//
// bwd_prep_kernel  -- per (chunk, value head): q^, k^ (the forward's bit-exact
//   normalisation), G, P (L = diag(beta) P), Aqk, T = (I+L)^-1, A = T
//   diag(beta), E = exp(G) k^, W = A E, U = A v, Qg, Kg, gamma = exp(G_last),
//   written to the chunk's record in the workspace.
// bwd_carry_fwd_kernel -- per (sequence, value head, 32 state columns), in
//   chunk order: stores each chunk's entering state S (transposed) and
//   Vnew = U - W S, then S = gamma S + Kg^T Vnew.
// bwd_carry_rev_kernel -- same split, chunks in reverse, with dS' the
//   gradient of the chunk's exiting state (starting from d_final_state):
//   stores dS' (transposed), dVnew = Aqk^T dO + Kg dS', then
//   dS' = gamma dS' + Qg^T dO - W^T dVnew; the last one is d_initial_state.
// bwd_grad_kernel -- per (chunk, value head): dQg = dO S^T, dAqk = tril(dO
//   Vnew^T), dKg = Vnew dS'^T, dgamma = rowsum(dS' * S), dW = -dVnew S^T,
//   dA = tril(dVnew v^T + dW E^T), dv = A^T dVnew, dE = A^T dW,
//   dT = dA diag(beta), dL = -tril_strict(T^T dT T^T), dbeta from A and L,
//   then the gated sums through P and Aqk, dq^, dk^ and dG, and dg as the
//   reverse cumulative sum of dG within the chunk.
// bwd_norm_kernel -- per (token, Q/K head): dq^, dk^ summed over the value
//   heads that share the Q/K head (GQA), then through the L2 norm:
//   dx = dy / n - x (x . dy) / n^3 with n^2 = sum(x*x) + 1e-6.
//
// Gated sums: with Gam_ij[d] = exp(G_id - G_jd) (j <= i, so <= 1 for
// non-positive gates), Mk = diag(beta) dL and Mq = K^-1/2 dAqk,
//   RK_i = sum_{j<i} Mk_ij k_j Gam_ij     CK_j = sum_{i>j} Mk_ij k_i Gam_ij
//   RQ_i = sum_{j<=i} Mq_ij k_j Gam_ij    CQ_j = sum_{i>=j} Mq_ij q_i Gam_ij
//   dk^ += RK + CK + CQ, dq^ += RQ, dG += k^ RK + q^ RQ - k^ CK - k^ CQ.
#include "kda_device.h"
#include "kda_host.h"

#include <atomic>

namespace {

using kda::bf16f;

constexpr int C = 64;             // chunk size
constexpr int KD = kda::kHead;    // K == V == 128
constexpr int NTB = 256;          // threads per workgroup
constexpr int KP = KD + 4;        // LDS row stride of [C][KD] fp32 tiles (16-byte aligned rows)
constexpr int CP = C + 2;         // LDS row stride of [C][C] fp32 tiles
constexpr int SP = 33;            // LDS row stride of 32-column state slices
constexpr int NCOL = 32;          // state columns per carry workgroup
constexpr float kScale = 0.08838834764831845f;   // 128^-1/2

// Per-chunk record in the workspace (float offsets), one per (value head,
// chunk slot), slots numbered as in the forward: chunk c of sequence n is
// slot floor(first_token(n) / 64) + n + c.
constexpr int R_QN = 0;                     // [C][K] q^ (bf16 values)
constexpr int R_KN = R_QN + C * KD;         // [C][K] k^
constexpr int R_G = R_KN + C * KD;          // [C][K] G, inclusive prefix of g
constexpr int R_E = R_G + C * KD;           // [C][K] exp(G) k^
constexpr int R_W = R_E + C * KD;           // [C][K] A E
constexpr int R_U = R_W + C * KD;           // [C][V] A v
constexpr int R_QG = R_U + C * KD;          // [C][K] K^-1/2 q^ exp(G)
constexpr int R_KG = R_QG + C * KD;         // [C][K] k^ exp(G_last - G)
constexpr int R_P = R_KG + C * KD;          // [C][C] P_ij = sum_d k_id k_jd Gam_ij (j < i)
constexpr int R_AQK = R_P + C * C;          // [C][C] Aqk (j <= i)
constexpr int R_T = R_AQK + C * C;          // [C][C] (I + diag(beta) P)^-1
constexpr int R_A = R_T + C * C;            // [C][C] T diag(beta)
constexpr int R_GAM = R_A + C * C;          // [K] exp(G_last)
constexpr int R_ST = R_GAM + KD;            // [V][K] entering state, transposed
constexpr int R_VN = R_ST + KD * KD;        // [C][V] Vnew
constexpr int R_DST = R_VN + C * KD;        // [V][K] gradient of the exiting state, transposed
constexpr int R_DVN = R_DST + KD * KD;      // [C][V] dVnew
constexpr int REC = R_DVN + C * KD;         // floats per record
static_assert(REC % 4 == 0, "records stay 16-byte aligned");

struct BParams {
  const uint16_t* q;        // bf16 [tokens][H][K]
  const uint16_t* k;
  const uint16_t* v;        // bf16 [tokens][HV][V]
  const float* g;           // [tokens][HV][K]
  const uint16_t* beta;     // bf16 [tokens][HV]
  const float* s0;          // [N][HV][K][V] or null
  const int32_t* cu;        // [N+1] or null
  const uint16_t* dout;     // bf16 [tokens][HV][V]
  const float* dht;         // [N][HV][K][V] or null
  float* dq;                // [tokens][H][K]
  float* dk;
  float* dv;                // [tokens][HV][V]
  float* dg;                // [tokens][HV][K]
  float* dbeta;             // [tokens][HV]
  float* dh0;               // [N][HV][K][V] or null
  float* ws;                // records [HV][nslots][REC]
  float* dqh;               // [tokens][HV][K] dq^ per value head
  float* dkh;
  int64_t nslots;           // slots per value head
  int64_t tokens;
  int T, H, HV, N;
};

__device__ __forceinline__ void seq_range(const BParams& p, int n, int64_t& tok0, int& len) {
  if (p.cu) {
    tok0 = p.cu[n];
    len = p.cu[n + 1] - p.cu[n];
  } else {
    tok0 = int64_t(n) * p.T;
    len = p.T;
  }
}

__device__ __forceinline__ int64_t slot_base(const BParams& p, int n) {
  const int64_t tok0 = p.cu ? int64_t(p.cu[n]) : int64_t(n) * p.T;
  return tok0 / C + n;
}

// The sequence owning slot s and its chunk index, or -1 for a slot between
// sequences.
__device__ int slot_owner(const BParams& p, int64_t s, int& chunk) {
  int lo = 0, hi = p.N - 1;                 // largest n with slot_base(n) <= s
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (slot_base(p, mid) <= s) lo = mid; else hi = mid - 1;
  }
  int64_t tok0;
  int len;
  seq_range(p, lo, tok0, len);
  const int64_t c = s - slot_base(p, lo);
  if (c < 0 || c * C >= len) return -1;
  chunk = int(c);
  return lo;
}

__device__ __forceinline__ float* record(const BParams& p, int hv, int64_t slot) {
  return p.ws + (int64_t(hv) * p.nslots + slot) * REC;
}

// (i, j), j <= i, of lower-triangle pair index t (row-major over the triangle).
__device__ __forceinline__ void tri_pair(int t, int& i, int& j) {
  int r = int((sqrtf(8.0f * float(t) + 1.0f) - 1.0f) * 0.5f);
  while (r * (r + 1) / 2 > t) --r;
  while ((r + 1) * (r + 2) / 2 <= t) ++r;
  i = r;
  j = t - r * (r + 1) / 2;
}
constexpr int kPairs = C * (C + 1) / 2;

// Copy a [C][KD] fp32 tile from the record into LDS (row stride KP).
__device__ __forceinline__ void load_tile(float* dst, const float* src, int tid) {
  for (int u = tid; u < C * KD / 4; u += NTB) {
    const int r = u / (KD / 4), c4 = u - r * (KD / 4);
    *reinterpret_cast<float4*>(dst + r * KP + 4 * c4) = reinterpret_cast<const float4*>(src)[u];
  }
}

// --------------------------------------------------------------- prep
constexpr int PREP_LDS = (3 * C * KP + 2 * C * CP + C) * 4;

__global__ __launch_bounds__(NTB) void bwd_prep_kernel(BParams p) {
  extern __shared__ __align__(16) float smem[];
  float* sQ = smem;                 // q^, later E
  float* sK = sQ + C * KP;          // k^, later v
  float* sG = sK + C * KP;          // G
  float* sP = sG + C * KP;          // P, later A
  float* sT = sP + C * CP;          // T
  float* sB = sT + C * CP;          // beta

  const int64_t slot = blockIdx.x;
  const int hv = blockIdx.y;
  int c;
  const int n = slot_owner(p, slot, c);
  if (n < 0) return;
  int64_t tok0;
  int len;
  seq_range(p, n, tok0, len);
  const int64_t t0 = tok0 + int64_t(c) * C;
  const int nv = min(C, len - c * C);
  const int hq = hv / (p.HV / p.H);
  float* rec = record(p, hv, slot);
  const int tid = threadIdx.x;

  // q^ and k^: 16 rows per pass (16 lanes per row, 8 elements per lane);
  // rows 0..63 are q, 64..127 are k; rows past the chunk's end are zero.
  for (int pass = 0; pass < 2 * C / 16; ++pass) {
    const int r = pass * 16 + (tid >> 4);
    const int l16 = tid & 15;
    const bool isk = r >= C;
    const int tr = r & (C - 1);
    uint4 x = make_uint4(0u, 0u, 0u, 0u);
    if (tr < nv)
      x = *reinterpret_cast<const uint4*>((isk ? p.k : p.q) + ((t0 + tr) * p.H + hq) * KD + 8 * l16);
    const uint4 y = kda::l2norm_row16(x);
    const uint32_t w[4] = {y.x, y.y, y.z, y.w};
    float f[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = kda::bf16lo(w[e]);
      f[2 * e + 1] = kda::bf16hi(w[e]);
    }
    float* dl = (isk ? sK : sQ) + tr * KP + 8 * l16;
    float* dgl = rec + (isk ? R_KN : R_QN) + tr * KD + 8 * l16;
    *reinterpret_cast<float4*>(dl) = make_float4(f[0], f[1], f[2], f[3]);
    *reinterpret_cast<float4*>(dl + 4) = make_float4(f[4], f[5], f[6], f[7]);
    *reinterpret_cast<float4*>(dgl) = make_float4(f[0], f[1], f[2], f[3]);
    *reinterpret_cast<float4*>(dgl + 4) = make_float4(f[4], f[5], f[6], f[7]);
  }
  // G: inclusive prefix over the chunk's tokens (padding has g = 0).
  if (tid < KD) {
    float acc = 0.0f;
    for (int t = 0; t < C; ++t) {
      if (t < nv) acc += p.g[((t0 + t) * p.HV + hv) * KD + tid];
      sG[t * KP + tid] = acc;
      rec[R_G + t * KD + tid] = acc;
    }
  }
  if (tid < C) sB[tid] = tid < nv ? bf16f(p.beta[(t0 + tid) * p.HV + hv]) : 0.0f;
  __syncthreads();

  // P and Aqk over the lower triangle; zeros above it.
  for (int t = tid; t < kPairs; t += NTB) {
    int i, j;
    tri_pair(t, i, j);
    const float* ki = sK + i * KP;
    const float* kj = sK + j * KP;
    const float* qi = sQ + i * KP;
    const float* gi = sG + i * KP;
    const float* gj = sG + j * KP;
    float pk = 0.0f, pq = 0.0f;
    for (int d = 0; d < KD; ++d) {
      const float e = expf(gi[d] - gj[d]);
      const float kje = kj[d] * e;
      pk = fmaf(ki[d], kje, pk);
      pq = fmaf(qi[d], kje, pq);
    }
    const float pv = j < i ? pk : 0.0f;
    sP[i * CP + j] = pv;
    rec[R_P + i * C + j] = pv;
    rec[R_AQK + i * C + j] = kScale * pq;
  }
  for (int t = tid; t < C * C; t += NTB) {
    const int i = t / C, j = t - i * C;
    if (j > i) {
      sP[i * CP + j] = 0.0f;
      rec[R_P + t] = 0.0f;
      rec[R_AQK + t] = 0.0f;
    }
  }
  __syncthreads();

  // T = (I + diag(beta) P)^-1 by forward substitution, one column per thread.
  if (tid < C) {
    const int j = tid;
    for (int i = 0; i < C; ++i) {
      float tv;
      if (i < j) {
        tv = 0.0f;
      } else if (i == j) {
        tv = 1.0f;
      } else {
        float acc = 0.0f;
        for (int m = j; m < i; ++m) acc = fmaf(sP[i * CP + m], sT[m * CP + j], acc);
        tv = -sB[i] * acc;
      }
      sT[i * CP + j] = tv;
    }
  }
  __syncthreads();
  // A = T diag(beta) (into sP); T and A to the record.
  for (int t = tid; t < C * C; t += NTB) {
    const int i = t / C, j = t - i * C;
    const float tv = sT[i * CP + j];
    const float a = tv * sB[j];
    rec[R_T + t] = tv;
    rec[R_A + t] = a;
    sP[i * CP + j] = a;
  }
  if (tid < KD) rec[R_GAM + tid] = expf(sG[(C - 1) * KP + tid]);
  // Qg, Kg, E (E replaces q^ in LDS).
  for (int t = tid; t < C * KD; t += NTB) {
    const int i = t / KD, d = t - i * KD;
    const float gv = sG[i * KP + d];
    const float eg = expf(gv);
    const float kv = sK[i * KP + d];
    rec[R_QG + t] = kScale * sQ[i * KP + d] * eg;
    rec[R_KG + t] = kv * expf(sG[(C - 1) * KP + d] - gv);
    const float ev = eg * kv;
    rec[R_E + t] = ev;
    sQ[i * KP + d] = ev;
  }
  __syncthreads();
  // v (zero past the chunk's end) replaces k^ in LDS.
  for (int t = tid; t < C * KD; t += NTB) {
    const int i = t / KD, d = t - i * KD;
    sK[i * KP + d] = i < nv ? bf16f(p.v[((t0 + i) * p.HV + hv) * KD + d]) : 0.0f;
  }
  __syncthreads();
  // W = A E and U = A v (A lower triangular).
  {
    const int d = tid & (KD - 1);
    for (int i = tid >> 7; i < C; i += 2) {
      float w = 0.0f, u = 0.0f;
      for (int j = 0; j <= i; ++j) {
        const float a = sP[i * CP + j];
        w = fmaf(a, sQ[j * KP + d], w);
        u = fmaf(a, sK[j * KP + d], u);
      }
      rec[R_W + i * KD + d] = w;
      rec[R_U + i * KD + d] = u;
    }
  }
}

// --------------------------------------------------------------- carries
// Workgroup (column group cg, value head hv, sequence n) owns state columns
// 32 cg .. 32 cg + 31.  Thread t works on column j = t % 32.
constexpr int FWD_LDS = (KD * SP + 2 * C * KP + 2 * C * SP) * 4;
constexpr int REV_LDS = (KD * SP + C * CP + 3 * C * KP + 2 * C * SP + KD) * 4;
static_assert(FWD_LDS <= 160 * 1024 && REV_LDS <= 160 * 1024, "LDS budget");

__global__ __launch_bounds__(NTB) void bwd_carry_fwd_kernel(BParams p) {
  extern __shared__ __align__(16) float smem[];
  float* sS = smem;                 // [K][32] state slice
  float* sW = sS + KD * SP;         // [C][K]
  float* sKg = sW + C * KP;         // [C][K]
  float* sU = sKg + C * KP;         // [C][32]
  float* sV = sU + C * SP;          // [C][32] Vnew

  const int cg = blockIdx.x, hv = blockIdx.y, n = blockIdx.z;
  const int c0 = cg * NCOL;
  const int tid = threadIdx.x;
  const int j = tid & (NCOL - 1);
  const int rg = tid >> 5;          // 0..7
  int64_t tok0;
  int len;
  seq_range(p, n, tok0, len);
  const int nch = (len + C - 1) / C;
  const int64_t sb = slot_base(p, n);

  for (int d = rg; d < KD; d += 8)
    sS[d * SP + j] = p.s0 ? p.s0[((int64_t(n) * p.HV + hv) * KD + d) * KD + c0 + j] : 0.0f;
  __syncthreads();

  for (int c = 0; c < nch; ++c) {
    float* rec = record(p, hv, sb + c);
    // Entering state, transposed: ST[v][d] for this group's columns v.
    for (int t = tid; t < NCOL * KD; t += NTB) {
      const int vv = t / KD, d = t - vv * KD;
      rec[R_ST + (c0 + vv) * KD + d] = sS[d * SP + vv];
    }
    load_tile(sW, rec + R_W, tid);
    load_tile(sKg, rec + R_KG, tid);
    for (int i = rg; i < C; i += 8) sU[i * SP + j] = rec[R_U + i * KD + c0 + j];
    __syncthreads();
    // Vnew = U - W S.
    for (int i = rg; i < C; i += 8) {
      float acc = sU[i * SP + j];
      const float* w = sW + i * KP;
      for (int d = 0; d < KD; ++d) acc = fmaf(-w[d], sS[d * SP + j], acc);
      sV[i * SP + j] = acc;
      rec[R_VN + i * KD + c0 + j] = acc;
    }
    __syncthreads();
    // S = gamma S + Kg^T Vnew.
    float ns[KD / 8];
#pragma unroll
    for (int m = 0; m < KD / 8; ++m) {
      const int d = rg + 8 * m;
      float acc = rec[R_GAM + d] * sS[d * SP + j];
      for (int i = 0; i < C; ++i) acc = fmaf(sKg[i * KP + d], sV[i * SP + j], acc);
      ns[m] = acc;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < KD / 8; ++m) sS[(rg + 8 * m) * SP + j] = ns[m];
    __syncthreads();
  }
}

__global__ __launch_bounds__(NTB) void bwd_carry_rev_kernel(BParams p) {
  extern __shared__ __align__(16) float smem[];
  float* sD = smem;                 // [K][32] dS' slice
  float* sAqk = sD + KD * SP;       // [C][C]
  float* sKg = sAqk + C * CP;       // [C][K]
  float* sQg = sKg + C * KP;        // [C][K]
  float* sW = sQg + C * KP;         // [C][K]
  float* sO = sW + C * KP;          // [C][32] dO
  float* sV = sO + C * SP;          // [C][32] dVnew
  float* sGam = sV + C * SP;        // [K]

  const int cg = blockIdx.x, hv = blockIdx.y, n = blockIdx.z;
  const int c0 = cg * NCOL;
  const int tid = threadIdx.x;
  const int j = tid & (NCOL - 1);
  const int rg = tid >> 5;
  int64_t tok0;
  int len;
  seq_range(p, n, tok0, len);
  const int nch = (len + C - 1) / C;
  const int64_t sb = slot_base(p, n);
  const int64_t sh = (int64_t(n) * p.HV + hv) * KD;

  for (int d = rg; d < KD; d += 8) sD[d * SP + j] = p.dht ? p.dht[(sh + d) * KD + c0 + j] : 0.0f;
  __syncthreads();

  for (int c = nch - 1; c >= 0; --c) {
    float* rec = record(p, hv, sb + c);
    const int nv = min(C, len - c * C);
    const int64_t t0 = tok0 + int64_t(c) * C;
    for (int t = tid; t < NCOL * KD; t += NTB) {
      const int vv = t / KD, d = t - vv * KD;
      rec[R_DST + (c0 + vv) * KD + d] = sD[d * SP + vv];
    }
    for (int t = tid; t < C * C; t += NTB) {
      const int i = t / C, jj = t - i * C;
      sAqk[i * CP + jj] = rec[R_AQK + t];
    }
    load_tile(sKg, rec + R_KG, tid);
    load_tile(sQg, rec + R_QG, tid);
    load_tile(sW, rec + R_W, tid);
    for (int i = rg; i < C; i += 8)
      sO[i * SP + j] = i < nv ? bf16f(p.dout[((t0 + i) * p.HV + hv) * KD + c0 + j]) : 0.0f;
    if (tid < KD) sGam[tid] = rec[R_GAM + tid];
    __syncthreads();
    // dVnew = Aqk^T dO + Kg dS'.
    for (int i = rg; i < C; i += 8) {
      float acc = 0.0f;
      for (int m = i; m < C; ++m) acc = fmaf(sAqk[m * CP + i], sO[m * SP + j], acc);
      const float* kg = sKg + i * KP;
      for (int d = 0; d < KD; ++d) acc = fmaf(kg[d], sD[d * SP + j], acc);
      sV[i * SP + j] = acc;
      rec[R_DVN + i * KD + c0 + j] = acc;
    }
    __syncthreads();
    // dS = gamma dS' + Qg^T dO - W^T dVnew.
    float nd[KD / 8];
#pragma unroll
    for (int m = 0; m < KD / 8; ++m) {
      const int d = rg + 8 * m;
      float acc = sGam[d] * sD[d * SP + j];
      for (int i = 0; i < C; ++i) {
        acc = fmaf(sQg[i * KP + d], sO[i * SP + j], acc);
        acc = fmaf(-sW[i * KP + d], sV[i * SP + j], acc);
      }
      nd[m] = acc;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < KD / 8; ++m) sD[(rg + 8 * m) * SP + j] = nd[m];
    __syncthreads();
  }
  if (p.dh0)
    for (int d = rg; d < KD; d += 8) p.dh0[(sh + d) * KD + c0 + j] = sD[d * SP + j];
}

// --------------------------------------------------------------- gradients
// Thread t owns channel (or value column) d = t % 128 and rows
// i = t / 128 + 2 m, m = 0..31, of every [C][128] quantity.
constexpr int NR = C / 2;
constexpr int GRAD_LDS = (2 * C * KP + 5 * C * CP + 2 * C + KD) * 4;
static_assert(GRAD_LDS <= 160 * 1024, "LDS budget");
static_assert(2 * C * CP == C * KP, "A and T together alias one [C][KP] tile");

__global__ __launch_bounds__(NTB) void bwd_grad_kernel(BParams p) {
  extern __shared__ __align__(16) float smem[];
  float* sX = smem;                 // dO, then dW, then q^
  float* sZ = sX + C * KP;          // Vnew, then dVnew, then G
  float* sA = sZ + C * KP;          // A        } later k^ ([C][KP] over both)
  float* sT = sA + C * CP;          // T        }
  float* sM1 = sT + C * CP;         // dAqk
  float* sM2 = sM1 + C * CP;        // dA, then dT, then dL
  float* sM3 = sM2 + C * CP;        // dT T^T
  float* sB = sM3 + C * CP;         // beta
  float* sDB = sB + C;              // dbeta
  float* sGl = sDB + C;             // dG_last
  float* sKn = sA;

  const int64_t slot = blockIdx.x;
  const int hv = blockIdx.y;
  int c;
  const int n = slot_owner(p, slot, c);
  if (n < 0) return;
  int64_t tok0;
  int len;
  seq_range(p, n, tok0, len);
  const int64_t t0 = tok0 + int64_t(c) * C;
  const int nv = min(C, len - c * C);
  const float* rec = record(p, hv, slot);
  const int tid = threadIdx.x;
  const int d = tid & (KD - 1);
  const int hr = tid >> 7;

  float dq[NR], dk[NR], dG[NR];
#pragma unroll
  for (int m = 0; m < NR; ++m) dq[m] = dk[m] = dG[m] = 0.0f;
  float dgl = 0.0f;   // this thread's share of dG_last[d]

  // dO (zero past the chunk's end) and Vnew; A, T, beta.
  for (int t = tid; t < C * KD; t += NTB) {
    const int i = t / KD, e = t - i * KD;
    sX[i * KP + e] = i < nv ? bf16f(p.dout[((t0 + i) * p.HV + hv) * KD + e]) : 0.0f;
  }
  load_tile(sZ, rec + R_VN, tid);
  for (int t = tid; t < C * C; t += NTB) {
    const int i = t / C, j = t - i * C;
    sA[i * CP + j] = rec[R_A + t];
    sT[i * CP + j] = rec[R_T + t];
  }
  if (tid < C) {
    sB[tid] = tid < nv ? bf16f(p.beta[(t0 + tid) * p.HV + hv]) : 0.0f;
    sDB[tid] = 0.0f;
  }
  __syncthreads();

  // dQg = dO S^T: dq^ += K^-1/2 dQg exp(G), dG += dQg Qg.
  {
    float acc[NR];
#pragma unroll
    for (int m = 0; m < NR; ++m) acc[m] = 0.0f;
    for (int vv = 0; vv < KD; ++vv) {
      const float s = rec[R_ST + vv * KD + d];
#pragma unroll
      for (int m = 0; m < NR; ++m) acc[m] = fmaf(sX[(hr + 2 * m) * KP + vv], s, acc[m]);
    }
#pragma unroll
    for (int m = 0; m < NR; ++m) {
      const int i = hr + 2 * m;
      dq[m] = fmaf(kScale * acc[m], expf(rec[R_G + i * KD + d]), dq[m]);
      dG[m] = fmaf(acc[m], rec[R_QG + i * KD + d], dG[m]);
    }
  }
  // dAqk = tril(dO Vnew^T).
  for (int t = tid; t < C * C; t += NTB) {
    const int i = t / C, j = t - i * C;
    float acc = 0.0f;
    if (j <= i) {
      const float* a = sX + i * KP;
      const float* b = sZ + j * KP;
      for (int e = 0; e < KD; ++e) acc = fmaf(a[e], b[e], acc);
    }
    sM1[i * CP + j] = acc;
  }
  // dKg = Vnew dS'^T: dk^ += dKg exp(G_last - G), dG -= dKg Kg, dG_last += dKg Kg.
  {
    float acc[NR];
#pragma unroll
    for (int m = 0; m < NR; ++m) acc[m] = 0.0f;
    for (int vv = 0; vv < KD; ++vv) {
      const float s = rec[R_DST + vv * KD + d];
#pragma unroll
      for (int m = 0; m < NR; ++m) acc[m] = fmaf(sZ[(hr + 2 * m) * KP + vv], s, acc[m]);
    }
    const float gl = rec[R_G + (C - 1) * KD + d];
#pragma unroll
    for (int m = 0; m < NR; ++m) {
      const int i = hr + 2 * m;
      const float kg = rec[R_KG + i * KD + d];
      dk[m] = fmaf(acc[m], expf(gl - rec[R_G + i * KD + d]), dk[m]);
      dG[m] = fmaf(-acc[m], kg, dG[m]);
      dgl = fmaf(acc[m], kg, dgl);
    }
  }
  // dgamma = rowsum(dS' * S): dG_last += dgamma gamma.
  if (hr == 0) {
    float acc = 0.0f;
    for (int vv = 0; vv < KD; ++vv) acc = fmaf(rec[R_DST + vv * KD + d], rec[R_ST + vv * KD + d], acc);
    dgl = fmaf(acc, rec[R_GAM + d], dgl);
  }
  __syncthreads();   // dO and Vnew are consumed

  // dVnew; dW = -dVnew S^T (into sX).
  load_tile(sZ, rec + R_DVN, tid);
  __syncthreads();
  {
    float acc[NR];
#pragma unroll
    for (int m = 0; m < NR; ++m) acc[m] = 0.0f;
    for (int vv = 0; vv < KD; ++vv) {
      const float s = rec[R_ST + vv * KD + d];
#pragma unroll
      for (int m = 0; m < NR; ++m) acc[m] = fmaf(sZ[(hr + 2 * m) * KP + vv], s, acc[m]);
    }
#pragma unroll
    for (int m = 0; m < NR; ++m) sX[(hr + 2 * m) * KP + d] = -acc[m];
  }
  __syncthreads();
  // dA = tril(dVnew v^T + dW E^T).
  for (int t = tid; t < C * C; t += NTB) {
    const int i = t / C, j = t - i * C;
    float acc = 0.0f;
    if (j <= i) {
      const float* dvn = sZ + i * KP;
      const float* dw = sX + i * KP;
      const float* ej = rec + R_E + j * KD;
      if (j < nv) {
        const uint16_t* vj = p.v + ((t0 + j) * p.HV + hv) * KD;
        for (int e = 0; e < KD; ++e) acc = fmaf(dvn[e], bf16f(vj[e]), acc);
      }
      for (int e = 0; e < KD; ++e) acc = fmaf(dw[e], ej[e], acc);
    }
    sM2[i * CP + j] = acc;
  }
  // dv = A^T dVnew; dE = A^T dW: dk^ += dE exp(G), dG += dE E.
#pragma unroll
  for (int m = 0; m < NR; ++m) {
    const int j = hr + 2 * m;
    float av = 0.0f, ae = 0.0f;
    for (int i = j; i < C; ++i) {
      const float a = sA[i * CP + j];
      av = fmaf(a, sZ[i * KP + d], av);
      ae = fmaf(a, sX[i * KP + d], ae);
    }
    if (j < nv) p.dv[((t0 + j) * p.HV + hv) * KD + d] = av;
    dk[m] = fmaf(ae, expf(rec[R_G + j * KD + d]), dk[m]);
    dG[m] = fmaf(ae, rec[R_E + j * KD + d], dG[m]);
  }
  __syncthreads();
  // dbeta_j += sum_i dA_ij T_ij; then dT = dA diag(beta).
  if (tid < C) {
    const int j = tid;
    float acc = 0.0f;
    for (int i = j; i < C; ++i) acc = fmaf(sM2[i * CP + j], sT[i * CP + j], acc);
    sDB[j] += acc;
  }
  __syncthreads();
  for (int t = tid; t < C * C; t += NTB) {
    const int i = t / C, j = t - i * C;
    sM2[i * CP + j] *= sB[j];
  }
  __syncthreads();
  // X = dT T^T (both lower triangular).
  for (int t = tid; t < C * C; t += NTB) {
    const int i = t / C, mm = t - i * C;
    float acc = 0.0f;
    const int lim = min(i, mm);
    for (int j = 0; j <= lim; ++j) acc = fmaf(sM2[i * CP + j], sT[mm * CP + j], acc);
    sM3[i * CP + mm] = acc;
  }
  __syncthreads();
  // dL = -tril_strict(T^T X) (into sM2).
  for (int t = tid; t < C * C; t += NTB) {
    const int a = t / C, b = t - a * C;
    float acc = 0.0f;
    if (b < a)
      for (int i = a; i < C; ++i) acc = fmaf(sT[i * CP + a], sM3[i * CP + b], acc);
    sM2[a * CP + b] = -acc;
  }
  __syncthreads();
  // dbeta_i += sum_j dL_ij P_ij.
  if (tid < C) {
    const int i = tid;
    float acc = 0.0f;
    for (int j = 0; j < i; ++j) acc = fmaf(sM2[i * CP + j], rec[R_P + i * C + j], acc);
    sDB[i] += acc;
  }
  // k^, q^, G for the gated sums (k^ over A and T, which are consumed).
  load_tile(sKn, rec + R_KN, tid);
  load_tile(sX, rec + R_QN, tid);
  load_tile(sZ, rec + R_G, tid);
  __syncthreads();
  // Gated sums through P (Mk = diag(beta) dL) and Aqk (Mq = K^-1/2 dAqk).
#pragma unroll
  for (int m = 0; m < NR; ++m) {
    const int i = hr + 2 * m;
    const float gi = sZ[i * KP + d];
    const float ki = sKn[i * KP + d];
    const float qi = sX[i * KP + d];
    const float bi = sB[i];
    float rk = 0.0f, rq = 0.0f;
    for (int j = 0; j <= i; ++j) {   // row forms
      const float e = expf(gi - sZ[j * KP + d]) * sKn[j * KP + d];
      rk = fmaf(bi * sM2[i * CP + j], e, rk);
      rq = fmaf(kScale * sM1[i * CP + j], e, rq);
    }
    float ck = 0.0f, cq = 0.0f;
    for (int r = i; r < C; ++r) {     // column forms (row i as the column index)
      const float e = expf(sZ[r * KP + d] - gi);
      ck = fmaf(sB[r] * sM2[r * CP + i], sKn[r * KP + d] * e, ck);
      cq = fmaf(kScale * sM1[r * CP + i], sX[r * KP + d] * e, cq);
    }
    dk[m] += rk + ck + cq;
    dq[m] += rq;
    dG[m] += ki * rk + qi * rq - ki * ck - ki * cq;
  }
  // dG_last onto the last row, then dg as the reverse prefix of dG.
  __syncthreads();
  if (hr == 1) sGl[d] = dgl;
  __syncthreads();
  if (hr == 0) sGl[d] += dgl;
  __syncthreads();
#pragma unroll
  for (int m = 0; m < NR; ++m) {
    const int i = hr + 2 * m;
    float v = dG[m];
    if (i == C - 1) v += sGl[d];
    sX[i * KP + d] = v;
    if (i < nv) {
      p.dqh[((t0 + i) * p.HV + hv) * KD + d] = dq[m];
      p.dkh[((t0 + i) * p.HV + hv) * KD + d] = dk[m];
    }
  }
  __syncthreads();
  if (hr == 0) {
    float acc = 0.0f;
    for (int i = C - 1; i >= 0; --i) {
      acc += sX[i * KP + d];
      if (i < nv) p.dg[((t0 + i) * p.HV + hv) * KD + d] = acc;
    }
  }
  if (tid < nv) p.dbeta[(t0 + tid) * p.HV + hv] = sDB[tid];
}

// --------------------------------------------------------------- norm
// One 64-lane wave per (token, Q/K head, q or k) row; lane l holds elements
// l and l + 64.
__global__ __launch_bounds__(NTB) void bwd_norm_kernel(BParams p) {
  const int64_t row = int64_t(blockIdx.x) * (NTB / 64) + (threadIdx.x >> 6);
  const int64_t rows = p.tokens * p.H;
  if (row >= 2 * rows) return;
  const bool isk = row >= rows;
  const int64_t r = isk ? row - rows : row;   // token * H + h
  const int64_t tok = r / p.H;
  const int h = int(r - tok * p.H);
  const int lane = threadIdx.x & 63;
  const int grp = p.HV / p.H;
  const uint16_t* x = (isk ? p.k : p.q) + r * KD;
  const float* dy = (isk ? p.dkh : p.dqh) + (tok * p.HV + int64_t(h) * grp) * KD;
  float xv[2], gv[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int dd = lane + 64 * e;
    xv[e] = bf16f(x[dd]);
    float s = 0.0f;
    for (int u = 0; u < grp; ++u) s += dy[u * KD + dd];
    gv[e] = s;
  }
  float ss = xv[0] * xv[0] + xv[1] * xv[1];
  float xd = xv[0] * gv[0] + xv[1] * gv[1];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    ss += __shfl_xor(ss, off, 64);
    xd += __shfl_xor(xd, off, 64);
  }
  const float nrm = sqrtf(ss + 1e-6f);
  const float inv = 1.0f / nrm;
  const float c3 = xd * inv * inv * inv;
  float* out = (isk ? p.dk : p.dq) + r * KD;
#pragma unroll
  for (int e = 0; e < 2; ++e) out[lane + 64 * e] = gv[e] * inv - xv[e] * c3;
}

// Raise a kernel's dynamic-LDS limit once per device.
constexpr int kMaxDevices = 64;
template <typename Kern>
int set_lds(Kern kern, int bytes, std::atomic<bool> (&done)[kMaxDevices]) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KDA_ERR_HIP;
  if (!done[dev].load(std::memory_order_acquire)) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            bytes) != hipSuccess)
      return KDA_ERR_HIP;
    done[dev].store(true, std::memory_order_release);
  }
  return KDA_OK;
}

int64_t slots_per_head(int64_t tokens, int64_t nseq) { return tokens / C + nseq + 1; }

}  // namespace

extern "C" size_t kda_chunk_backward_workspace_size(int32_t B, int32_t T, int32_t H, int32_t HV, int32_t Kd,
                                                    int32_t Vd, int32_t num_seqs) {
  (void)H;
  if (B < 1 || T < 0 || HV < 1 || Kd != KD || Vd != KD) return 0;
  const int64_t nseq = num_seqs > 0 ? num_seqs : B;
  const int64_t tokens = int64_t(B) * T;
  return size_t(slots_per_head(tokens, nseq) * HV) * REC * 4 + size_t(tokens) * HV * KD * 4 * 2;
}

extern "C" int kda_chunk_backward(const void* q, const void* k, const void* v, const float* g, const void* beta,
                                  const float* initial_state, const int32_t* cu_seqlens, int32_t num_seqs,
                                  int32_t B, int32_t T, int32_t H, int32_t HV, int32_t Kd, int32_t Vd,
                                  const void* d_out, const float* d_final_state, float* dq, float* dk, float* dv,
                                  float* dg, float* dbeta, float* d_initial_state, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (B < 1 || T < 0 || H < 1 || HV < 1 || HV % H != 0) return KDA_ERR_SHAPE;
  if (Kd != KD || Vd != KD) return KDA_ERR_UNSUPPORTED;
  if (cu_seqlens && (B != 1 || num_seqs < 1)) return KDA_ERR_SHAPE;
  const int64_t nseq = cu_seqlens ? num_seqs : B;
  const int64_t tokens = int64_t(B) * T;
  if (tokens > 0 && (!q || !k || !v || !g || !beta || !d_out || !dq || !dk || !dv || !dg || !dbeta))
    return KDA_ERR_NULL;
  if (!kda::aligned16(q) || !kda::aligned16(k) || !kda::aligned16(v) || !kda::aligned16(g) ||
      !kda::aligned16(d_out) || !kda::aligned16(dq) || !kda::aligned16(dk) || !kda::aligned16(dv) ||
      !kda::aligned16(dg) || !kda::aligned16(workspace))
    return KDA_ERR_ALIGN;
  const size_t need = kda_chunk_backward_workspace_size(B, T, H, HV, Kd, Vd, int32_t(nseq));
  if (!workspace) return KDA_ERR_NULL;
  if (workspace_bytes < need) return KDA_ERR_WORKSPACE;
  const int64_t nslots = slots_per_head(tokens, nseq);
  if (nslots > 0x7fffffff || HV > 65535 || nseq > 65535 || 2 * tokens * H / (NTB / 64) + 1 > 0x7fffffff)
    return KDA_ERR_SHAPE;

  BParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.g = g;
  p.beta = static_cast<const uint16_t*>(beta);
  p.s0 = initial_state;
  p.cu = cu_seqlens;
  p.dout = static_cast<const uint16_t*>(d_out);
  p.dht = d_final_state;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.dg = dg;
  p.dbeta = dbeta;
  p.dh0 = d_initial_state;
  p.ws = static_cast<float*>(workspace);
  p.dqh = p.ws + nslots * HV * REC;
  p.dkh = p.dqh + tokens * HV * KD;
  p.nslots = nslots;
  p.tokens = tokens;
  p.T = T;
  p.H = H;
  p.HV = HV;
  p.N = int(nseq);

  static std::atomic<bool> prep_set[kMaxDevices], fwd_set[kMaxDevices], rev_set[kMaxDevices],
      grad_set[kMaxDevices];
  if (set_lds(&bwd_prep_kernel, PREP_LDS, prep_set) != KDA_OK ||
      set_lds(&bwd_carry_fwd_kernel, FWD_LDS, fwd_set) != KDA_OK ||
      set_lds(&bwd_carry_rev_kernel, REV_LDS, rev_set) != KDA_OK ||
      set_lds(&bwd_grad_kernel, GRAD_LDS, grad_set) != KDA_OK)
    return KDA_ERR_HIP;
  hipStream_t s = kda::as_stream(stream);
  const dim3 chunks = dim3(unsigned(nslots), unsigned(HV));
  const dim3 carries = dim3(KD / NCOL, unsigned(HV), unsigned(nseq));
  hipLaunchKernelGGL(bwd_prep_kernel, chunks, dim3(NTB), PREP_LDS, s, p);
  int st = kda::launch_status();
  if (st != KDA_OK) return st;
  hipLaunchKernelGGL(bwd_carry_fwd_kernel, carries, dim3(NTB), FWD_LDS, s, p);
  st = kda::launch_status();
  if (st != KDA_OK) return st;
  hipLaunchKernelGGL(bwd_carry_rev_kernel, carries, dim3(NTB), REV_LDS, s, p);
  st = kda::launch_status();
  if (st != KDA_OK) return st;
  if (tokens == 0) return KDA_OK;
  hipLaunchKernelGGL(bwd_grad_kernel, chunks, dim3(NTB), GRAD_LDS, s, p);
  st = kda::launch_status();
  if (st != KDA_OK) return st;
  const int64_t rows = 2 * tokens * H;
  hipLaunchKernelGGL(bwd_norm_kernel, dim3(unsigned((rows + NTB / 64 - 1) / (NTB / 64))), dim3(NTB), 0, s, p);
  return kda::launch_status();
}
