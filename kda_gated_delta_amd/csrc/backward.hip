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
// Workgroup barriers order LDS only (kda::lds_barrier): no data crosses
// threads through global memory inside a kernel, and the plain barrier
// would also wait for every outstanding global load and store.
//
// Everything runs in float32.  Five kernels (four when every Q/K head has
// one value head), split where the method splits
// (chunk-local work is chunk-parallel, the carries are sequential per
// (sequence, value head) and column-parallel, since column v of the state
// only ever meets column v of the values):
//
// bwd_prep_kernel  -- per (chunk, value head): q^, k^ (the forward's bit-exact
//   normalisation), G, P (L = diag(beta) P), Aqk, T = (I+L)^-1, A = T
//   diag(beta), E = exp(G) k^, W = A E, U = A v, Qg, Kg, gamma = exp(G_last),
//   written to the chunk's record in the workspace.
// bwd_carry_fwd_kernel -- per (sequence, value head, 64 state columns), in
//   chunk order: stores each chunk's entering state S ([K][V], as the carry
//   holds it; the gradient kernel transposes it while staging) and
//   Vnew = U - W S (transposed), then S = gamma S + Kg^T Vnew.
// bwd_carry_rev_kernel -- same split, chunks in reverse, with dS' the
//   gradient of the chunk's exiting state (starting from d_final_state):
//   stores dS' ([K][V]) and dVnew = Aqk^T dO + Kg dS' (transposed), then
//   dS' = gamma dS' + Qg^T dO - W^T dVnew; the last one is d_initial_state.
// bwd_grad_kernel -- per (chunk, value head): dQg = dO S^T, dAqk = tril(dO
//   Vnew^T), dKg = Vnew dS'^T, dgamma = rowsum(dS' * S), dW = -dVnew S^T,
//   dA = tril(dVnew v^T + dW E^T), dv = A^T dVnew, dE = A^T dW,
//   dT = dA diag(beta), dL = -tril_strict(T^T dT T^T), dbeta from A and L,
//   then the gated sums through P and Aqk, dq^, dk^ and dG, and dg as the
//   reverse cumulative sum of dG within the chunk; with one value head per
//   Q/K head, also the L2 norm's backward below on its own dq^ and dk^.
// bwd_norm_kernel -- per (token, Q/K head), only when Q/K heads are shared
//   (GQA): dq^, dk^ summed over the value heads that share the Q/K head,
//   then through the L2 norm: dx = dy / n - x (x . dy) / n^3 with
//   n^2 = sum(x*x) + 1e-6.
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
constexpr int NCOL = 64;          // state columns per carry workgroup
constexpr float kScale = 0.08838834764831845f;   // 128^-1/2
constexpr float kLog2e = 1.4426950408889634f;

// 2^x by the hardware instruction (results below 2^-126 flush to zero;
// they only ever scale terms of sums, so the loss is below 1e-38 absolute).
// G is kept in log2 units (G log2 e), so exp(G_i - G_j) = 2^(G2_i - G2_j).
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Per-chunk record in the workspace (float offsets), one per (value head,
// chunk slot), slots numbered as in the forward: chunk c of sequence n is
// slot floor(first_token(n) / 64) + n + c.
constexpr int R_QN = 0;                     // [C][K] q^ as bf16 (two per float slot)
constexpr int R_KN = R_QN + C * KD / 2;     // [C][K] k^ as bf16
constexpr int R_G = R_KN + C * KD / 2;      // [C][K] G log2(e), G the inclusive prefix of g
constexpr int R_W = R_G + C * KD;           // [C][K] A E (E = exp(G) k^ is formed where it is needed)
constexpr int R_U = R_W + C * KD;           // [C][V] A v
constexpr int R_QG = R_U + C * KD;          // [C][K] K^-1/2 q^ exp(G)
constexpr int R_KG = R_QG + C * KD;         // [C][K] k^ exp(G_last - G)
constexpr int R_P = R_KG + C * KD;          // [C][C] P_ij = sum_d k_id k_jd Gam_ij (j < i)
constexpr int R_AQK = R_P + C * C;          // [C][C] Aqk (j <= i)
constexpr int R_T = R_AQK + C * C;          // [C][C] (I + diag(beta) P)^-1
constexpr int R_A = R_T + C * C;            // [C][C] T diag(beta)
constexpr int R_GAM = R_A + C * C;          // [K] exp(G_last)
constexpr int R_ST = R_GAM + KD;            // [K][V] entering state
constexpr int R_DST = R_ST + KD * KD;       // [K][V] gradient of the exiting state
constexpr int R_WT = R_DST + KD * KD;       // [K][C] W transposed
constexpr int R_KGT = R_WT + KD * C;        // [K][C] Kg transposed
constexpr int R_ET = R_KGT + KD * C;        // [K][C] E transposed
constexpr int R_VNT = R_ET + KD * C;        // [V][C] Vnew transposed
constexpr int R_DVNT = R_VNT + KD * C;      // [V][C] dVnew transposed
constexpr int REC = R_DVNT + KD * C;        // floats per record
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
  void* dq;                 // [tokens][H][K]   float32, or bf16 when obf
  void* dk;
  void* dv;                 // [tokens][HV][V]  float32, or bf16 when obf
  float* dg;                // [tokens][HV][K]
  void* dbeta;              // [tokens][HV]     float32, or bf16 when obf
  float* dh0;               // [N][HV][K][V] or null
  float* ws;                // records [HV][nslots][REC]
  float* dqh;               // [tokens][HV][K] dq^ per value head
  float* dkh;
  int64_t nslots;           // slots per value head
  int64_t tokens;
  int T, H, HV, N;
  int obf;                  // dq, dk, dv, dbeta stored as bf16 (nearest-even), else float32
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

// --------------------------------------------------------------- helpers
constexpr int LQ = C + 4;         // LDS row stride of [*][C] fp32 tiles (16-byte aligned rows)

// 16-byte values kept across phases are native vectors: locals of HIP's
// float4 struct type in arrays were not promoted to registers.
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4f ldg4(const float* p) { return *reinterpret_cast<const v4f*>(p); }
__device__ __forceinline__ void sts4(float* p, v4f v) { *reinterpret_cast<v4f*>(p) = v; }

// Copy rows [r0, r0 + rows) of a [*][cols] fp32 record matrix, columns
// [c0, c0 + w), into LDS with row stride ld (all multiples of 4).
template <int NTH = NTB>
__device__ __forceinline__ void load_rows(float* dst, int ld, const float* src, int cols, int r0, int rows, int c0,
                                          int w, int tid) {
  const int q4 = w / 4;
  for (int u = tid; u < rows * q4; u += NTH) {
    const int r = u / q4, c4 = u - r * q4;
    *reinterpret_cast<float4*>(dst + r * ld + 4 * c4) =
        *reinterpret_cast<const float4*>(src + (r0 + r) * cols + c0 + 4 * c4);
  }
}

__device__ __forceinline__ float4 lds4(const float* p) { return *reinterpret_cast<const float4*>(p); }

// acc[r][c] += a[r] * b[c] for a 4-row (or 8-row, two calls) tile.
__device__ __forceinline__ void fma4x4(float (*acc)[4], const float4 a, const float4 b, float sign) {
  const float av[4] = {sign * a.x, sign * a.y, sign * a.z, sign * a.w};
  const float bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = fmaf(av[r], bv[c], acc[r][c]);
}

__device__ __forceinline__ void st8(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

__device__ __forceinline__ float2 lds2(const float* p) { return *reinterpret_cast<const float2*>(p); }


__device__ __forceinline__ void ld4(const float* p, float* v) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
}

__device__ __forceinline__ void st4(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

// Gradient outputs that take their input's dtype: element `idx` of a
// float32 array, or of a bf16 array (the same float32 value rounded to
// nearest-even) when `obf` is set.  idx is a multiple of 4 for put4.
__device__ __forceinline__ void put4(void* base, int64_t idx, const float* v, int obf) {
  if (obf)
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + idx) =
        make_uint2(kda::pack_bf16(v[0], v[1]), kda::pack_bf16(v[2], v[3]));
  else
    st4(static_cast<float*>(base) + idx, v);
}
__device__ __forceinline__ void put1(void* base, int64_t idx, float v, int obf) {
  if (obf)
    static_cast<uint16_t*>(base)[idx] = uint16_t(kda::pack_bf16(v, 0.0f));
  else
    static_cast<float*>(base)[idx] = v;
}

// fp32 MFMA (v_mfma_f32_16x16x4_f32), twice the rate of plain fp32 VALU code
// here: lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16] and holds
// D[4 (l / 16) + r][l % 16] in register r (checked on the chip).
typedef float f32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4v mfma4(float a, float b, f32x4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// --------------------------------------------------------------- prep
// 512 threads.  [C][128] results in 4x4 tiles (rows 4 (t / 32), columns
// 4 (t % 32)); P and Aqk in 4x4 blocks of (i, j) pairs (below).
constexpr int NTP = 512;
constexpr int XS = 20;            // row stride of the T solve's [16][16] X tiles
constexpr int PREP_LDS = (3 * C * KP + 2 * C * LQ + C + 3 * 16 * XS) * 4;

__global__ __launch_bounds__(NTP) void bwd_prep_kernel(BParams p) {
  extern __shared__ __align__(16) float smem[];
  float* sQ = smem;                 // q^, later E
  float* sK = sQ + C * KP;          // k^, later v
  float* sG = sK + C * KP;          // G (log2 units)
  float* sP = sG + C * KP;          // P [C][LQ]
  float* sAT = sP + C * LQ;         // A^T [C][LQ]
  float* sB = sAT + C * LQ;         // beta
  float* sXs = sB + C;              // three [16][XS] tiles for the T solve

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
  const int i0 = 4 * (tid >> 5), d0 = 4 * (tid & 31);

  // Raw inputs first, all loads in flight together: the q and k rows of
  // the four normalisation passes (32 rows per pass, 16 lanes per row, 8
  // elements per lane; rows 0..63 are q, 64..127 are k) and this thread's
  // four 16-byte pieces of g.  Rows past the chunk's end are zero.
  uint4 xr[2 * C / 32];
#pragma unroll
  for (int pass = 0; pass < 2 * C / 32; ++pass) {
    const int r = pass * 32 + (tid >> 4);
    const int tr = r & (C - 1);
    xr[pass] = make_uint4(0u, 0u, 0u, 0u);
    if (tr < nv)
      xr[pass] = *reinterpret_cast<const uint4*>((r >= C ? p.k : p.q) + ((t0 + tr) * p.H + hq) * KD + 8 * (tid & 15));
  }
  v4u vraw[C * KD / 8 / NTP];   // v: row u / 16, 8 values from column 8 (u % 16)
#pragma unroll
  for (int k = 0; k < C * KD / 8 / NTP; ++k) {
    const int u = tid + NTP * k, row = u >> 4, c8 = u & 15;
    vraw[k] = row < nv ? *reinterpret_cast<const v4u*>(p.v + ((t0 + row) * p.HV + hv) * KD + 8 * c8)
                       : v4u{0u, 0u, 0u, 0u};
  }
  v4f graw[C * KD / 4 / NTP];
#pragma unroll
  for (int k = 0; k < C * KD / 4 / NTP; ++k) {
    const int u = tid + NTP * k, row = u / (KD / 4), c4 = u - row * (KD / 4);
    graw[k] = row < nv ? ldg4(p.g + ((t0 + row) * p.HV + hv) * KD + 4 * c4) : v4f{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int pass = 0; pass < 2 * C / 32; ++pass) {
    const int r = pass * 32 + (tid >> 4);
    const int l16 = tid & 15;
    const bool isk = r >= C;
    const int tr = r & (C - 1);
    const uint4 y = kda::l2norm_row16(xr[pass]);
    const uint32_t w[4] = {y.x, y.y, y.z, y.w};
    float f[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = kda::bf16lo(w[e]);
      f[2 * e + 1] = kda::bf16hi(w[e]);
    }
    st8((isk ? sK : sQ) + tr * KP + 8 * l16, f);
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(rec + (isk ? R_KN : R_QN)) + tr * KD + 8 * l16) = y;
  }
  // G: inclusive prefix of g over the chunk's tokens (padding has g = 0),
  // kept in log2 units: prefixes within four 16-row blocks per channel,
  // then the totals of the earlier blocks.
#pragma unroll
  for (int k = 0; k < C * KD / 4 / NTP; ++k) {
    const int u = tid + NTP * k, row = u / (KD / 4), c4 = u - row * (KD / 4);
    sts4(sG + row * KP + 4 * c4, graw[k]);
  }
  kda::lds_barrier();
  {
    const int d = tid & (KD - 1), blk = tid >> 7;
    float pre[16];
    float acc = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc += sG[(16 * blk + r) * KP + d];
      pre[r] = acc;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sG[(16 * blk + r) * KP + d] = pre[r];
    kda::lds_barrier();
    float off = 0.0f;
    for (int b = 0; b < blk; ++b) off += sG[(16 * b + 15) * KP + d];
    kda::lds_barrier();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float g2 = (pre[r] + off) * kLog2e;
      sG[(16 * blk + r) * KP + d] = g2;
      rec[R_G + (16 * blk + r) * KD + d] = g2;
    }
  }
  if (tid < C) sB[tid] = tid < nv ? bf16f(p.beta[(t0 + tid) * p.HV + hv]) : 0.0f;
  kda::lds_barrier();

  // P (j < i) and Aqk (j <= i).  The six 16x16 tiles below the diagonal
  // run on MFMA in waves 0-2, two tiles each ((1,0) (3,2); (2,0) (2,1);
  // (3,0) (3,1)): with r the first row of tile row I, exp(G_i - G_j) =
  // exp(G_i - G_r) exp(G_r - G_j), both <= 1, so P's tile is the product of
  // k^_i exp(G_i - G_r) and k^_j exp(G_r - G_j) over the channels (Aqk's with
  // q^_i), each lane forming its operand values from LDS (shared by the two
  // tiles when they share I); in k-step s of a 16-channel block, lane group
  // g takes channel 4 s + g (rows 4 mod 64 words apart, so the groups read
  // disjoint banks).  The four diagonal tiles run on VALU in waves 3-7, in
  // 4x4 blocks of pairs with eight lanes per block (channel eighths): lanes
  // 192..383 take the 24 blocks below their diagonals, split around the
  // block's first row a0 as above; lanes 384..511 take the 16 blocks on the
  // diagonal, formed directly (j <= i only).  Partial sums are combined
  // with register-only DPP moves.
  {
    if (tid < 192) {
      const int wave = tid >> 6, lg = (tid >> 4) & 3, l16 = tid & 15;
      const int I0 = wave == 0 ? 1 : wave + 1, J0 = 0;
      const int I1 = wave == 0 ? 3 : wave + 1, J1 = wave == 0 ? 2 : 1;
      const bool share = I0 == I1;
      const int ra = 16 * I0, rb = 16 * I1;
      f32x4v ap0 = {0.f, 0.f, 0.f, 0.f}, aq0 = ap0, ap1 = ap0, aq1 = ap0;
#pragma unroll 2
      for (int kb = 0; kb < KD; kb += 16)
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const int d = kb + 4 * s4 + lg;
          const float ga = sG[ra * KP + d];
          const float fa = ex2(sG[(ra + l16) * KP + d] - ga);
          const float gb = share ? ga : sG[rb * KP + d];
          const float fb = share ? fa : ex2(sG[(rb + l16) * KP + d] - gb);
          const float b0 = sK[(16 * J0 + l16) * KP + d] * ex2(ga - sG[(16 * J0 + l16) * KP + d]);
          const float b1 = sK[(16 * J1 + l16) * KP + d] * ex2(gb - sG[(16 * J1 + l16) * KP + d]);
          ap0 = mfma4(sK[(ra + l16) * KP + d] * fa, b0, ap0);
          aq0 = mfma4(sQ[(ra + l16) * KP + d] * fa, b0, aq0);
          ap1 = mfma4(sK[(rb + l16) * KP + d] * fb, b1, ap1);
          aq1 = mfma4(sQ[(rb + l16) * KP + d] * fb, b1, aq1);
        }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row0 = ra + 4 * lg + r, row1 = rb + 4 * lg + r;
        const int j0 = 16 * J0 + l16, j1 = 16 * J1 + l16;
        sP[row0 * LQ + j0] = ap0[r];
        rec[R_P + row0 * C + j0] = ap0[r];
        rec[R_AQK + row0 * C + j0] = kScale * aq0[r];
        sP[row1 * LQ + j1] = ap1[r];
        rec[R_P + row1 * C + j1] = ap1[r];
        rec[R_AQK + row1 * C + j1] = kScale * aq1[r];
      }
    } else {
      const int u = tid - 192;
      const bool below = u < 192, diag = !below;
      int bi, bj;
      if (below) {
        tri_pair((u >> 3) % 6, bi, bj);
        ++bi;
        bi += 4 * ((u >> 3) / 6);
        bj += 4 * ((u >> 3) / 6);
      } else {
        bi = bj = (u - 192) >> 3;
      }
      const int d_lo = (KD / 8) * (u & 7), d_hi = d_lo + KD / 8;
      const int a0 = 4 * bi, b0 = 4 * bj;
      float pk[4][4] = {}, pq[4][4] = {};
      if (below) {
        for (int d = d_lo; d < d_hi; d += 4) {
          float4 gi[4], gj[4], ki[4], kj[4], qi[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            gi[r] = lds4(sG + (a0 + r) * KP + d);
            gj[r] = lds4(sG + (b0 + r) * KP + d);
            ki[r] = lds4(sK + (a0 + r) * KP + d);
            kj[r] = lds4(sK + (b0 + r) * KP + d);
            qi[r] = lds4(sQ + (a0 + r) * KP + d);
          }
          float4 fr[4], fc[4];
          fr[0] = make_float4(1.f, 1.f, 1.f, 1.f);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (r > 0)
              fr[r] = make_float4(ex2(gi[r].x - gi[0].x), ex2(gi[r].y - gi[0].y), ex2(gi[r].z - gi[0].z),
                                  ex2(gi[r].w - gi[0].w));
            fc[r] = make_float4(ex2(gi[0].x - gj[r].x) * kj[r].x, ex2(gi[0].y - gj[r].y) * kj[r].y,
                                ex2(gi[0].z - gj[r].z) * kj[r].z, ex2(gi[0].w - gj[r].w) * kj[r].w);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float4 a = make_float4(ki[r].x * fr[r].x, ki[r].y * fr[r].y, ki[r].z * fr[r].z, ki[r].w * fr[r].w);
            const float4 b = make_float4(qi[r].x * fr[r].x, qi[r].y * fr[r].y, qi[r].z * fr[r].z, qi[r].w * fr[r].w);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              pk[r][q] = fmaf(a.x, fc[q].x, fmaf(a.y, fc[q].y, fmaf(a.z, fc[q].z, fmaf(a.w, fc[q].w, pk[r][q]))));
              pq[r][q] = fmaf(b.x, fc[q].x, fmaf(b.y, fc[q].y, fmaf(b.z, fc[q].z, fmaf(b.w, fc[q].w, pq[r][q]))));
            }
          }
        }
      } else if (diag) {
        for (int d = d_lo; d < d_hi; d += 4) {
          float4 gi[4], ki[4], qi[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            gi[r] = lds4(sG + (a0 + r) * KP + d);
            ki[r] = lds4(sK + (a0 + r) * KP + d);
            qi[r] = lds4(sQ + (a0 + r) * KP + d);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int q = 0; q <= r; ++q) {   // no positive exponent is formed
              const float k0 = ki[q].x * ex2(gi[r].x - gi[q].x), k1 = ki[q].y * ex2(gi[r].y - gi[q].y);
              const float k2 = ki[q].z * ex2(gi[r].z - gi[q].z), k3 = ki[q].w * ex2(gi[r].w - gi[q].w);
              pk[r][q] = fmaf(ki[r].x, k0, fmaf(ki[r].y, k1, fmaf(ki[r].z, k2, fmaf(ki[r].w, k3, pk[r][q]))));
              pq[r][q] = fmaf(qi[r].x, k0, fmaf(qi[r].y, k1, fmaf(qi[r].z, k2, fmaf(qi[r].w, k3, pq[r][q]))));
            }
        }
      }
      // Sum over each block's eight lanes: neighbours, pairs, mirrored quads.
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          pk[r][q] += __uint_as_float(kda::dpp32<kda::kDppXor1>(__float_as_uint(pk[r][q])));
          pq[r][q] += __uint_as_float(kda::dpp32<kda::kDppXor1>(__float_as_uint(pq[r][q])));
          pk[r][q] += __uint_as_float(kda::dpp32<kda::kDppXor2>(__float_as_uint(pk[r][q])));
          pq[r][q] += __uint_as_float(kda::dpp32<kda::kDppXor2>(__float_as_uint(pq[r][q])));
          pk[r][q] += __uint_as_float(kda::dpp32<kda::kDppHalfMirror>(__float_as_uint(pk[r][q])));
          pq[r][q] += __uint_as_float(kda::dpp32<kda::kDppHalfMirror>(__float_as_uint(pq[r][q])));
        }
      if ((u & 7) == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = a0 + r;
          float pv[4], av[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int j = b0 + q;
            pv[q] = j < i ? pk[r][q] : 0.0f;
            av[q] = j <= i ? kScale * pq[r][q] : 0.0f;
          }
          const float4 p4 = make_float4(pv[0], pv[1], pv[2], pv[3]);
          *reinterpret_cast<float4*>(sP + i * LQ + b0) = p4;
          *reinterpret_cast<float4*>(rec + R_P + i * C + b0) = p4;
          *reinterpret_cast<float4*>(rec + R_AQK + i * C + b0) = make_float4(av[0], av[1], av[2], av[3]);
        }
      }
    }
    // The 120 4x4 blocks above the diagonal are zero: one row of one block
    // per lane.
    constexpr int kBelow = (C / 4) * (C / 4 - 1) / 2;
    for (int t = tid; t < 4 * kBelow; t += NTP) {
      int ui, uj;
      tri_pair(t >> 2, uj, ui);
      ++uj;
      const int i = 4 * ui + (t & 3), j0u = 4 * uj;
      const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
      *reinterpret_cast<float4*>(sP + i * LQ + j0u) = z;
      *reinterpret_cast<float4*>(rec + R_P + i * C + j0u) = z;
      *reinterpret_cast<float4*>(rec + R_AQK + i * C + j0u) = z;
    }
  }
  kda::lds_barrier();

  // T = (I + L)^-1 with L = diag(beta) P (strictly lower), blocked by 16
  // rows: the four diagonal blocks by forward substitution, then the blocks
  // below one block diagonal at a time, T_IJ = -T_II X with
  // X = diag(beta_I) sum_{J <= K < I} P_IK T_KJ, both products on MFMA.
  // T is kept transposed in sAT; at the end it goes to the record as T and
  // A = T diag(beta), and sAT is scaled to A^T.
  {
    // Diagonal blocks: lanes 8j .. 8j+7 own column j (block D = j / 16),
    // lane part p holding the block's local rows 2p and 2p+1; row i's sum
    // over the block's earlier rows is split by part and completed across
    // the eight lanes with register-only DPP moves.  (P is strictly lower
    // and T starts at zero, so the sums need no bounds.)
    const int j = tid >> 3, part = tid & 7, rb = 16 * (j >> 4), jl = j & 15;
    float t0v = 0.0f, t1v = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float2 pp = lds2(sP + (rb + i) * LQ + rb + 2 * part);
      float acc = fmaf(pp.y, t1v, pp.x * t0v);
      acc += __uint_as_float(kda::dpp32<kda::kDppXor1>(__float_as_uint(acc)));
      acc += __uint_as_float(kda::dpp32<kda::kDppXor2>(__float_as_uint(acc)));
      acc += __uint_as_float(kda::dpp32<kda::kDppHalfMirror>(__float_as_uint(acc)));
      const float tv = i == jl ? 1.0f : -sB[rb + i] * acc;
      if (part == (i >> 1)) {
        if (i & 1)
          t1v = tv;
        else
          t0v = tv;
      }
    }
    *reinterpret_cast<float2*>(sAT + j * LQ + rb + 2 * part) = make_float2(t0v, t1v);
    for (int u = tid; u < C * C; u += NTP) {   // T above its diagonal blocks is zero
      const int jj = u / C, ii = u - jj * C;
      if ((ii >> 4) < (jj >> 4)) sAT[jj * LQ + ii] = 0.0f;
    }
    kda::lds_barrier();
    // Blocks (J + lev, J): wave J takes one.  X's k-step s of a 16-block
    // takes k = 4 s + g in lane group g (P rows and T^T rows are read along
    // k); T_II X's takes k = s + 4 g (T^T and X read across k).  Either way
    // the four groups read disjoint banks.
    const int wave = tid >> 6, lg = (tid >> 4) & 3, l16 = tid & 15;
    for (int lev = 1; lev < 4; ++lev) {
      const bool act = wave < 4 - lev;
      const int J = wave, I = wave + lev;
      if (act) {
        f32x4v x = {0.f, 0.f, 0.f, 0.f};
        for (int kb = 16 * J; kb < 16 * I; kb += 16)
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4) {
            const int k = kb + 4 * s4 + lg;
            x = mfma4(sP[(16 * I + l16) * LQ + k], sAT[(16 * J + l16) * LQ + k], x);
          }
#pragma unroll
        for (int r = 0; r < 4; ++r) sXs[(16 * J + 4 * lg + r) * XS + l16] = sB[16 * I + 4 * lg + r] * x[r];
      }
      kda::lds_barrier();
      if (act) {
        f32x4v y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const int k = s4 + 4 * lg;
          y = mfma4(sAT[(16 * I + k) * LQ + 16 * I + l16], sXs[(16 * J + k) * XS + l16], y);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) sAT[(16 * J + l16) * LQ + 16 * I + 4 * lg + r] = -y[r];
      }
      kda::lds_barrier();
    }
    // T and A = T diag(beta) to the record, row by row from T^T.
    {
      const int i = tid >> 3, j8 = 8 * (tid & 7);
      float tv[8], av[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        tv[e] = sAT[(j8 + e) * LQ + i];
        av[e] = tv[e] * sB[j8 + e];
      }
      st8(rec + R_T + i * C + j8, tv);
      st8(rec + R_A + i * C + j8, av);
    }
    kda::lds_barrier();
    for (int u = tid; u < C * C; u += NTP) {   // A^T = diag(beta) T^T
      const int jj = u / C, ii = u - jj * C;
      sAT[jj * LQ + ii] *= sB[jj];
    }
  }
  if (tid < KD) rec[R_GAM + tid] = ex2(sG[(C - 1) * KP + tid]);
  // Qg, Kg, E over this thread's 4x4 tile (E replaces q^ in LDS; the
  // transposed copies are written four rows at a time).
  {
    float gl[4];
    ld4(sG + (C - 1) * KP + d0, gl);
    float kgt[4][4], et[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + r;
      float gv[4], kv[4], qv[4], qg[4], kg[4], ev[4];
      ld4(sG + i * KP + d0, gv);
      ld4(sK + i * KP + d0, kv);
      ld4(sQ + i * KP + d0, qv);
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const float eg = ex2(gv[cc]);
        qg[cc] = kScale * qv[cc] * eg;
        kg[cc] = kv[cc] * ex2(gl[cc] - gv[cc]);
        ev[cc] = eg * kv[cc];
        kgt[cc][r] = kg[cc];
        et[cc][r] = ev[cc];
      }
      st4(rec + R_QG + i * KD + d0, qg);
      st4(rec + R_KG + i * KD + d0, kg);
      st4(sQ + i * KP + d0, ev);
    }
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      st4(rec + R_KGT + (d0 + cc) * C + i0, kgt[cc]);
      st4(rec + R_ET + (d0 + cc) * C + i0, et[cc]);
    }
  }
  kda::lds_barrier();
  // v (zero past the chunk's end) replaces k^ in LDS.
#pragma unroll
  for (int k = 0; k < C * KD / 8 / NTP; ++k) {
    const int u = tid + NTP * k, row = u >> 4, c8 = u & 15;
    const uint32_t w[4] = {vraw[k].x, vraw[k].y, vraw[k].z, vraw[k].w};
    float f[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = kda::bf16lo(w[e]);
      f[2 * e + 1] = kda::bf16hi(w[e]);
    }
    st8(sK + row * KP + 8 * c8, f);
  }
  kda::lds_barrier();
  // W = A E and U = A v (A lower triangular: j <= i0 + 3 suffices).
  {
    float w[4][4] = {}, u[4][4] = {};
    for (int j = 0; j <= i0 + 3; ++j) {
      const float4 a = lds4(sAT + j * LQ + i0);
      fma4x4(w, a, lds4(sQ + j * KP + d0), 1.0f);
      fma4x4(u, a, lds4(sK + j * KP + d0), 1.0f);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      st4(rec + R_W + (i0 + r) * KD + d0, w[r]);
      st4(rec + R_U + (i0 + r) * KD + d0, u[r]);
    }
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
      *reinterpret_cast<float4*>(rec + R_WT + (d0 + cc) * C + i0) = make_float4(w[0][cc], w[1][cc], w[2][cc], w[3][cc]);
  }
}

// --------------------------------------------------------------- carries
// Workgroup (column group cg, value head hv, sequence n) owns state columns
// 64 cg .. 64 cg + 63, with 512 threads (two waves per SIMD).  Every
// product runs on fp32 MFMA in 16x16 output tiles, several tiles per wave
// sharing their A operand, with operands read from LDS layouts whose
// 16-lane groups touch consecutive words; in k-step s of each 16-wide
// block of the contraction, lane group g takes k = s + 4 g, so that with
// row strides of 4 mod 64 words the four groups read disjoint banks.
constexpr int SQ = NCOL + 4;      // LDS row stride of [rows][64-column] tiles
constexpr int NTC = 512;          // threads per carry workgroup
constexpr int FWD_LDS = (2 * KD * SQ + C * KP + C * SQ + KD) * 4;
constexpr int REV_LDS = (2 * KD * SQ + 3 * C * SQ + KD) * 4;
static_assert(FWD_LDS <= 160 * 1024 && REV_LDS <= 160 * 1024, "LDS budget");
static_assert(KD * SQ >= 2 * (C / 2) * KP, "two half tiles of Qg and W fit where Kg^T was");

// Both carries load the operands of the next chunk step into registers
// while the current step computes, so that their latency overlaps the
// products.  Thread t carries the 16-byte pieces t, t + 512, ... of each
// matrix in row-major order.

__global__ __launch_bounds__(NTC) void bwd_carry_fwd_kernel(BParams p) {
  extern __shared__ __align__(16) float smem[];
  float* sS = smem;                 // [K][64] state slice
  float* sWT = sS + KD * SQ;        // [K][C] W^T
  float* sKg = sWT + KD * SQ;       // [C][K] Kg
  float* sV = sKg + C * KP;         // [C][64] U, then Vnew
  float* sGam = sV + C * SQ;        // [K]

  const int cg = blockIdx.x, hv = blockIdx.y, n = blockIdx.z;
  const int c0 = cg * NCOL;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lg = (tid >> 4) & 3, l16 = tid & 15;   // MFMA lane roles
  int64_t tok0;
  int len;
  seq_range(p, n, tok0, len);
  const int nch = (len + C - 1) / C;
  const int64_t sb = slot_base(p, n);
  const int64_t sh = (int64_t(n) * p.HV + hv) * KD;

  for (int u = tid; u < KD * NCOL / 4; u += NTC) {
    const int d = u / (NCOL / 4), c4 = u - d * (NCOL / 4);
    *reinterpret_cast<float4*>(sS + d * SQ + 4 * c4) =
        p.s0 ? *reinterpret_cast<const float4*>(p.s0 + (sh + d) * KD + c0 + 4 * c4) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  v4f pwt[4], pkg[4], pu[2];      // W^T [K][C], Kg [C][K], U [C][64 columns]
  float pgam;                     // exp(G_last)[t % K]
  auto fetch = [&](const float* r) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      pwt[k] = ldg4(r + R_WT + 4 * (tid + NTC * k));
      pkg[k] = ldg4(r + R_KG + 4 * (tid + NTC * k));
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int u = tid + NTC * k, rr = u / (NCOL / 4), c4 = u - rr * (NCOL / 4);
      pu[k] = ldg4(r + R_U + rr * KD + c0 + 4 * c4);
    }
    pgam = r[R_GAM + (tid & (KD - 1))];
  };
  if (nch > 0) fetch(record(p, hv, sb));
  kda::lds_barrier();

  for (int c = 0; c < nch; ++c) {
    float* rec = record(p, hv, sb + c);
    // Entering state, this group's columns, 16 bytes per store.
#pragma unroll
    for (int k = 0; k < KD * NCOL / 4 / NTC; ++k) {
      const int u = tid + NTC * k, d = u / (NCOL / 4), c4 = u - d * (NCOL / 4);
      *reinterpret_cast<float4*>(rec + R_ST + d * KD + c0 + 4 * c4) = lds4(sS + d * SQ + 4 * c4);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int u = tid + NTC * k;
      const int rw = u / (C / 4), cw = u - rw * (C / 4);
      sts4(sWT + rw * SQ + 4 * cw, pwt[k]);
      const int rk = u / (KD / 4), ck = u - rk * (KD / 4);
      sts4(sKg + rk * KP + 4 * ck, pkg[k]);
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int u = tid + NTC * k, r = u / (NCOL / 4), c4 = u - r * (NCOL / 4);
      sts4(sV + r * SQ + 4 * c4, pu[k]);
    }
    if (tid < KD) sGam[tid] = pgam;
    kda::lds_barrier();
    fetch(record(p, hv, sb + min(c + 1, nch - 1)));   // next step (the last re-reads its own)
    // Vnew = U - W S on MFMA: wave w owns token block ib = w / 2 and column
    // blocks 2 (w % 2), 2 (w % 2) + 1 (two 16x16 tiles sharing A = W).
    {
      const int ib = wave >> 1, jb0 = 2 * (wave & 1);
      f32x4v acc[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t][r] = sV[(16 * ib + 4 * lg + r) * SQ + 16 * (jb0 + t) + l16];
#pragma unroll 4
      for (int ks = 0; ks < KD / 4; ++ks) {
        const int d = 16 * (ks >> 2) + (ks & 3) + 4 * lg;   // lane groups on disjoint banks
        const float a = -sWT[d * SQ + 16 * ib + l16];
        acc[0] = mfma4(a, sS[d * SQ + 16 * jb0 + l16], acc[0]);
        acc[1] = mfma4(a, sS[d * SQ + 16 * (jb0 + 1) + l16], acc[1]);
      }
      kda::lds_barrier();   // every wave has read its U tiles before Vnew overwrites them
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int j = 16 * (jb0 + t) + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * ib + 4 * lg + r;
          sV[i * SQ + j] = acc[t][r];
        }
        *reinterpret_cast<f32x4v*>(rec + R_VNT + (c0 + j) * C + 16 * ib + 4 * lg) = acc[t];
      }
    }
    kda::lds_barrier();
    // S = gamma S + Kg^T Vnew on MFMA: wave w owns state rows 16 w .. +15,
    // all four column blocks (A = Kg^T shared).
    {
      f32x4v acc[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d = 16 * wave + 4 * lg + r;
          acc[t][r] = sGam[d] * sS[d * SQ + 16 * t + l16];
        }
#pragma unroll 4
      for (int ks = 0; ks < C / 4; ++ks) {
        const int i = 16 * (ks >> 2) + (ks & 3) + 4 * lg;
        const float a = sKg[i * KP + 16 * wave + l16];
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = mfma4(a, sV[i * SQ + 16 * t + l16], acc[t]);
      }
      kda::lds_barrier();   // every wave has read S before it is overwritten
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) sS[(16 * wave + 4 * lg + r) * SQ + 16 * t + l16] = acc[t][r];
    }
    kda::lds_barrier();
  }
}

__global__ __launch_bounds__(NTC) void bwd_carry_rev_kernel(BParams p) {
  extern __shared__ __align__(16) float smem[];
  float* sD = smem;                 // [K][64] dS' slice
  float* sKgT = sD + KD * SQ;       // [K][C] Kg^T; later half tiles of Qg and W
  float* sAqk = sKgT + KD * SQ;     // [C][C] Aqk
  float* sO = sAqk + C * SQ;        // [C][64] dO
  float* sV = sO + C * SQ;          // [C][64] dVnew
  float* sGam = sV + C * SQ;        // [K]
  float* sQh = sKgT;                // [C/2][K] half of Qg
  float* sWh = sKgT + (C / 2) * KP; // [C/2][K] half of W

  const int cg = blockIdx.x, hv = blockIdx.y, n = blockIdx.z;
  const int c0 = cg * NCOL;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lg = (tid >> 4) & 3, l16 = tid & 15;   // MFMA lane roles
  int64_t tok0;
  int len;
  seq_range(p, n, tok0, len);
  const int nch = (len + C - 1) / C;
  const int64_t sb = slot_base(p, n);
  const int64_t sh = (int64_t(n) * p.HV + hv) * KD;

  for (int u = tid; u < KD * NCOL / 4; u += NTC) {
    const int d = u / (NCOL / 4), c4 = u - d * (NCOL / 4);
    *reinterpret_cast<float4*>(sD + d * SQ + 4 * c4) =
        p.dht ? *reinterpret_cast<const float4*>(p.dht + (sh + d) * KD + c0 + 4 * c4) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  v4f pkgt[4], paqk[2], pqg[4], pw[4];      // Kg^T [K][C], Aqk [C][C], Qg and W [C][K]
  v4u pdo;                                   // d_out: row t / 8, 8 bf16 of this group's columns
  float pgam;
  // Rows past the chunk's end are clamped here and zeroed when stored to LDS.
  auto fetch_a = [&](const float* r, int64_t t0, int nv) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 4; ++k) pkgt[k] = ldg4(r + R_KGT + 4 * (tid + NTC * k));
#pragma unroll
    for (int k = 0; k < 2; ++k) paqk[k] = ldg4(r + R_AQK + 4 * (tid + NTC * k));
    const int rr = min(tid >> 3, nv - 1), c8 = tid & 7;
    pdo = *reinterpret_cast<const v4u*>(p.dout + ((t0 + rr) * p.HV + hv) * KD + c0 + 8 * c8);
    pgam = r[R_GAM + (tid & (KD - 1))];
  };
  auto fetch_b = [&](const float* r, int h) __attribute__((always_inline)) {   // pieces 2h, 2h + 1: rows 32h .. 32h + 31
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      pqg[2 * h + k] = ldg4(r + R_QG + 4 * (tid + NTC * (2 * h + k)));
      pw[2 * h + k] = ldg4(r + R_W + 4 * (tid + NTC * (2 * h + k)));
    }
  };
  if (nch > 0) {
    const float* r0 = record(p, hv, sb + nch - 1);
    fetch_a(r0, tok0 + int64_t(nch - 1) * C, len - (nch - 1) * C);
    fetch_b(r0, 0);
    fetch_b(r0, 1);
  }
  kda::lds_barrier();

  for (int c = nch - 1; c >= 0; --c) {
    float* rec = record(p, hv, sb + c);
    const int nv = min(C, len - c * C);
    const int cn = max(c - 1, 0);     // next step (the first chunk re-reads its own)
    const float* recn = record(p, hv, sb + cn);
#pragma unroll
    for (int k = 0; k < KD * NCOL / 4 / NTC; ++k) {   // dS', this group's columns
      const int u = tid + NTC * k, d = u / (NCOL / 4), c4 = u - d * (NCOL / 4);
      *reinterpret_cast<float4*>(rec + R_DST + d * KD + c0 + 4 * c4) = lds4(sD + d * SQ + 4 * c4);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int u = tid + NTC * k, rr = u / (C / 4), cc = u - rr * (C / 4);
      sts4(sKgT + rr * SQ + 4 * cc, pkgt[k]);
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int u = tid + NTC * k, rr = u / (C / 4), cc = u - rr * (C / 4);
      sts4(sAqk + rr * SQ + 4 * cc, paqk[k]);
    }
    {
      const int r = tid >> 3, c8 = tid & 7;
      const uint32_t w[4] = {pdo.x, pdo.y, pdo.z, pdo.w};
      float f[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[2 * e] = r < nv ? kda::bf16lo(w[e]) : 0.0f;
        f[2 * e + 1] = r < nv ? kda::bf16hi(w[e]) : 0.0f;
      }
      st8(sO + r * SQ + 8 * c8, f);
    }
    if (tid < KD) sGam[tid] = pgam;
    kda::lds_barrier();
    fetch_a(recn, tok0 + int64_t(cn) * C, min(C, len - cn * C));
    // dVnew = Aqk^T dO + Kg dS' on MFMA: wave w owns token block ib = w / 2
    // and column blocks 2 (w % 2), +1 (two tiles sharing A).  Aqk[m][i] = 0
    // for m < i, so the first product starts at m = 16 ib.
    {
      const int ib = wave >> 1, jb0 = 2 * (wave & 1);
      f32x4v acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll 2
      for (int ks = 4 * ib; ks < C / 4; ++ks) {
        const int m = 16 * (ks >> 2) + (ks & 3) + 4 * lg;
        const float a = sAqk[m * SQ + 16 * ib + l16];
        acc[0] = mfma4(a, sO[m * SQ + 16 * jb0 + l16], acc[0]);
        acc[1] = mfma4(a, sO[m * SQ + 16 * (jb0 + 1) + l16], acc[1]);
      }
#pragma unroll 4
      for (int ks = 0; ks < KD / 4; ++ks) {
        const int d = 16 * (ks >> 2) + (ks & 3) + 4 * lg;   // lane groups on disjoint banks
        const float a = sKgT[d * SQ + 16 * ib + l16];
        acc[0] = mfma4(a, sD[d * SQ + 16 * jb0 + l16], acc[0]);
        acc[1] = mfma4(a, sD[d * SQ + 16 * (jb0 + 1) + l16], acc[1]);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int j = 16 * (jb0 + t) + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * ib + 4 * lg + r;
          sV[i * SQ + j] = acc[t][r];
        }
        *reinterpret_cast<f32x4v*>(rec + R_DVNT + (c0 + j) * C + 16 * ib + 4 * lg) = acc[t];
      }
    }
    // dS = gamma dS' + Qg^T dO - W^T dVnew on MFMA: wave w owns state rows
    // 16 w .. +15 and all four column blocks, with Qg and W staged 32 rows
    // at a time where Kg^T was (pieces k = 2h, 2h+1 of each thread are rows
    // 32h .. 32h+31).
    f32x4v acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = 16 * wave + 4 * lg + r;
        acc[t][r] = sGam[d] * sD[d * SQ + 16 * t + l16];
      }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      kda::lds_barrier();   // Kg^T (or the previous half) is no longer read; dVnew is complete
#pragma unroll
      for (int k = 2 * h; k < 2 * h + 2; ++k) {
        const int u = tid + NTC * k - h * (C / 2) * (KD / 4);
        const int rr = u / (KD / 4), cc = u - rr * (KD / 4);
        sts4(sQh + rr * KP + 4 * cc, pqg[k]);
        sts4(sWh + rr * KP + 4 * cc, pw[k]);
      }
      fetch_b(recn, h);
      kda::lds_barrier();
#pragma unroll 2
      for (int ks = 0; ks < C / 8; ++ks) {
        const int i = 16 * (ks >> 2) + (ks & 3) + 4 * lg;   // row within the half
        const int ig = h * (C / 2) + i;            // token
        const float aq = sQh[i * KP + 16 * wave + l16];
        const float aw = -sWh[i * KP + 16 * wave + l16];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          acc[t] = mfma4(aq, sO[ig * SQ + 16 * t + l16], acc[t]);
          acc[t] = mfma4(aw, sV[ig * SQ + 16 * t + l16], acc[t]);
        }
      }
    }
    kda::lds_barrier();   // every wave has read dS' (and the halves) before dS overwrites it
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) sD[(16 * wave + 4 * lg + r) * SQ + 16 * t + l16] = acc[t][r];
    kda::lds_barrier();
  }
  if (p.dh0)
    for (int u = tid; u < KD * NCOL / 4; u += NTC) {
      const int d = u / (NCOL / 4), c4 = u - d * (NCOL / 4);
      *reinterpret_cast<float4*>(p.dh0 + (sh + d) * KD + c0 + 4 * c4) = lds4(sD + d * SQ + 4 * c4);
    }
}

// --------------------------------------------------------------- gradients
// 512 threads (two waves per SIMD: the LDS footprint allows one workgroup
// per compute unit, and the second wave hides the first one's latency).
// Every [C][128] quantity is owned in 4x4 tiles: thread t holds rows
// 4 (t / 32) .. +3 and columns 4 (t % 32) .. +3; the dense products run on
// fp32 MFMA in 16x16 tiles and come back to those 4x4 tiles through LDS
// where elementwise work follows.  dq^ and dG accumulate in memory only the
// owning thread touches, dk^ in that thread's registers.  LDS holds three
// [128][68] regions (R0-R2), one [64][132] region (R3) and one [64][68]
// region (R4); what each holds changes by phase (below).
constexpr int NTG = 512;
constexpr int R0_OFF = 0;
constexpr int R1_OFF = R0_OFF + KD * LQ;
constexpr int R2_OFF = R1_OFF + KD * LQ;
constexpr int R3_OFF = R2_OFF + KD * LQ;
constexpr int R4_OFF = R3_OFF + C * KP;
constexpr int SM_OFF = R4_OFF + C * LQ;
constexpr int GRAD_LDS = (SM_OFF + 2 * C + KD) * 4;
static_assert(GRAD_LDS <= 160 * 1024, "LDS budget");
static_assert(C * KP <= KD * LQ && 2 * C * LQ <= KD * LQ && C * LQ <= C * KP, "regions hold their alternates");
static_assert((C / 4) * KD <= C * KP, "dG_last partials fit in R3");

// One 16x16 tile (I, J) of X Y^T on MFMA over k in [k0, k1) (multiples of
// 16, k1 > k0), with both operands stored transposed in LDS ([k][*], row
// stride ld).  In k-step s of each 16-wide block, lane group g takes
// k = s + 4 g (row strides are 4 mod 64 words, so the groups read disjoint
// banks); the next block's operands are loaded while the current one's
// four products run.
__device__ __forceinline__ f32x4v tile_mfma(f32x4v acc, const float* xt, const float* yt, int ld, int I, int J,
                                            int k0, int k1, int lg, int l16) {
  const float* xp = xt + (k0 + 4 * lg) * ld + 16 * I + l16;
  const float* yp = yt + (k0 + 4 * lg) * ld + 16 * J + l16;
  float xa[4], ya[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    xa[s] = xp[s * ld];
    ya[s] = yp[s * ld];
  }
  for (int kb = k0; kb < k1; kb += 16) {
    const int step = kb + 16 < k1 ? 16 * ld : 0;   // the last block re-reads itself
    xp += step;
    yp += step;
    float xb[4], yb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      xb[s] = xp[s * ld];
      yb[s] = yp[s * ld];
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma4(xa[s], ya[s], acc);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      xa[s] = xb[s];
      ya[s] = yb[s];
    }
  }
  return acc;
}
// Lower 16x16 tiles (J <= I) of a [C][C] product X Y^T over k in [0, K):
// wave w takes tiles w and w + 8 (when below 10) in the order (0,0) (1,0)
// (1,1) (2,0) ...
__device__ __forceinline__ void tri_tile(int t, int& I, int& J) {
  I = (t >= 1) + (t >= 3) + (t >= 6);
  J = t - I * (I + 1) / 2;
}
__device__ __forceinline__ void tri_mfma(f32x4v (&acc)[2], const float* xt, const float* yt, int ld, int K,
                                         int wave, int lg, int l16) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = wave + 8 * h;
    if (t < 10) {
      int I, J;
      tri_tile(t, I, J);
      acc[h] = tile_mfma(acc[h], xt, yt, ld, I, J, 0, K, lg, l16);
    }
  }
}
// Writes the tiles tri_mfma computed into out ([C][C], stride ld), keeping
// column <= row on the diagonal tiles, and zeroes the tiles above them.
__device__ __forceinline__ void tri_store(float* out, int ld, const f32x4v (&acc)[2], int wave, int lg, int l16,
                                          int tid) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = wave + 8 * h;
    if (t >= 10) break;
    int I, J;
    tri_tile(t, I, J);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * I + 4 * lg + r, j = 16 * J + l16;
      out[i * ld + j] = (j <= i) ? acc[h][r] : 0.0f;
    }
  }
  for (int u = tid; u < C * C; u += NTG) {
    const int i = u / C, j = u - i * C;
    if ((j >> 4) > (i >> 4)) out[i * ld + j] = 0.0f;
  }
}

__global__ __launch_bounds__(NTG) void bwd_grad_kernel(BParams p) {
  extern __shared__ __align__(16) float smem[];
  float* R0 = smem + R0_OFF;
  float* R1 = smem + R1_OFF;
  float* R2 = smem + R2_OFF;
  float* R3 = smem + R3_OFF;
  float* R4 = smem + R4_OFF;
  float* sB = smem + SM_OFF;        // beta
  float* sDB = sB + C;              // dbeta
  float* sGl = sDB + C;             // dG_last

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
  float* rec = record(p, hv, slot);
  const int tid = threadIdx.x;
  const int rb = tid >> 5;
  const int i0 = 4 * rb, d0 = 4 * (tid & 31);          // 4x4 tile of a [C][128] quantity
  float* gdq = p.dqh + (t0 * p.HV + hv) * KD;
  float* gdk = p.dkh + (t0 * p.HV + hv) * KD;
  const int64_t rs = int64_t(p.HV) * KD;     // token stride of gdq, gdk
  float* gdG = rec + R_U;                    // the record's U field is no longer read
  // This thread's 4x4 tile of dk^ is carried across the three phases in
  // registers (zero for rows past the chunk's end); dq^ and dG go through
  // memory, as registers for them too would spill (measured: dk^ alone
  // 2.3% faster at B=1 H=HV=96 T=8192, results unchanged).
  v4f pdk[4];
  const bool fused = p.H == p.HV;            // normalisation backward at the end of this kernel

  // ---- phase 1: dQg = dO S^T, dW = -dVnew S^T, dKg = Vnew dS'^T (on
  // MFMA), dgamma, then dAqk = tril(dO Vnew^T).  R0 = dO^T, R1 = Vnew^T,
  // R2 = dVnew^T ([V][C]); R3 = 32 rows of S^T then 32 rows of dS'^T per
  // block, the next block loaded into registers while the current one is
  // used.  Wave w owns token tiles 2 (w % 2) .. +1 and state-row tiles
  // 2 (w / 2) .. +1 (16x16 each) of all three products.  In k-step s of a
  // 16-row block of v, lane group g takes v = s + 4 g: the operand rows'
  // strides are 4 mod 64 words, so the four groups read disjoint banks.
  // Block vb of S and dS' is their columns 32 vb .. +31 (stored [K][V]),
  // transposed into R3 as it is staged: thread piece u is row d = u / 8,
  // columns 4 (u % 8) .. +3 of the block.
  v4f pst[2], pdst[2];
  auto fetch_blk = [&](int vb) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int u = tid + NTG * k, d = u >> 3, c4 = u & 7;
      pst[k] = ldg4(rec + R_ST + d * KD + 32 * vb + 4 * c4);
      pdst[k] = ldg4(rec + R_DST + d * KD + 32 * vb + 4 * c4);
    }
  };
  // Every load of the prologue is issued before the first is used: dO
  // (bf16; row u / 16, 8 values from column 8 (u % 16)), Vnew^T, dVnew^T
  // ([V][C]) and the first block of S^T / dS'^T.
  v4u pdo[C * KD / 8 / NTG];
  v4f pvn[KD * C / 4 / NTG], pdvn[KD * C / 4 / NTG];
#pragma unroll
  for (int k = 0; k < C * KD / 8 / NTG; ++k) {
    const int u = tid + NTG * k, j = u >> 4, c8 = u & 15;
    pdo[k] = j < nv ? *reinterpret_cast<const v4u*>(p.dout + ((t0 + j) * p.HV + hv) * KD + 8 * c8) : v4u{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int k = 0; k < KD * C / 4 / NTG; ++k) {
    pvn[k] = ldg4(rec + R_VNT + 4 * (tid + NTG * k));
    pdvn[k] = ldg4(rec + R_DVNT + 4 * (tid + NTG * k));
  }
  fetch_blk(0);
  const float beta_t = tid < nv ? bf16f(p.beta[(t0 + tid) * p.HV + hv]) : 0.0f;
#pragma unroll
  for (int k = 0; k < C * KD / 8 / NTG; ++k) {
    const int u = tid + NTG * k, j = u >> 4, c8 = u & 15;
    const uint32_t w[4] = {pdo[k].x, pdo[k].y, pdo[k].z, pdo[k].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      R0[(8 * c8 + 2 * e) * LQ + j] = kda::bf16lo(w[e]);
      R0[(8 * c8 + 2 * e + 1) * LQ + j] = kda::bf16hi(w[e]);
    }
  }
#pragma unroll
  for (int k = 0; k < KD * C / 4 / NTG; ++k) {
    const int u = tid + NTG * k, row = u / (C / 4), c4 = u - row * (C / 4);
    sts4(R1 + row * LQ + 4 * c4, pvn[k]);
    sts4(R2 + row * LQ + 4 * c4, pdvn[k]);
  }
  if (tid < C) {
    sB[tid] = beta_t;
    sDB[tid] = 0.0f;
  }
  const int wave = tid >> 6, lg = (tid >> 4) & 3, l16 = tid & 15;   // MFMA lane roles
  const int it0 = 2 * (wave & 1), dt0 = 2 * (wave >> 1);
  f32x4v mq[2][2], mw[2][2], mk[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) mq[a][b] = mw[a][b] = mk[a][b] = f32x4v{0.f, 0.f, 0.f, 0.f};
  float dgp = 0.0f;   // dgamma partial: state row tid % 128, rows 8 (tid / 128) .. +7 of each block
  for (int vb = 0; vb < KD / 32; ++vb) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int u = tid + NTG * k, d = u >> 3, c4 = u & 7;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        R3[(4 * c4 + e) * KP + d] = pst[k][e];
        R3[(32 + 4 * c4 + e) * KP + d] = pdst[k][e];
      }
    }
    kda::lds_barrier();
    if (vb + 1 < KD / 32) fetch_blk(vb + 1);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int vl = 16 * (ks >> 2) + (ks & 3) + 4 * lg;   // row of the block
      const int vv = 32 * vb + vl;
      float bs[2], bd[2], ao[2], av[2], adv[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        bs[t] = R3[vl * KP + 16 * (dt0 + t) + l16];
        bd[t] = R3[(32 + vl) * KP + 16 * (dt0 + t) + l16];
        ao[t] = R0[vv * LQ + 16 * (it0 + t) + l16];
        av[t] = R1[vv * LQ + 16 * (it0 + t) + l16];
        adv[t] = R2[vv * LQ + 16 * (it0 + t) + l16];
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          mq[a][b] = mfma4(ao[a], bs[b], mq[a][b]);
          mw[a][b] = mfma4(adv[a], bs[b], mw[a][b]);
          mk[a][b] = mfma4(av[a], bd[b], mk[a][b]);
        }
    }
    {
      const int d = tid & (KD - 1), v8 = 8 * (tid >> 7);
#pragma unroll
      for (int u = 0; u < 8; ++u) dgp = fmaf(R3[(v8 + u) * KP + d], R3[(32 + v8 + u) * KP + d], dgp);
    }
    kda::lds_barrier();
  }
  // The epilogue's global operands (G, q^ and k^ rows of this thread's
  // tile, G_last, gamma), issued now so that they arrive during the round
  // trips.  Qg and Kg are formed from them as the recompute kernel forms
  // them, sharing the epilogue's exponentials, rather than read back.
  v4f egv[4];
  uint2 eqn[4], ekn[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    egv[r] = ldg4(rec + R_G + (i0 + r) * KD + d0);
    eqn[r] = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(rec + R_QN) + (i0 + r) * KD + d0);
    ekn[r] = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(rec + R_KN) + (i0 + r) * KD + d0);
  }
  const v4f egl = ldg4(rec + R_G + (C - 1) * KD + d0);
  const v4f egm = rb == 0 ? ldg4(rec + R_GAM + d0) : v4f{0.f, 0.f, 0.f, 0.f};
  // dgamma partials into R4 ([4][128]); dQg and dKg to this thread's 4x4
  // tiles through R3 (dW stays in MFMA order until phase 2).
  R4[(tid >> 7) * KD + (tid & (KD - 1))] = dgp;
  float aq[4][4], akg[4][4];
  auto to_tiles = [&](const f32x4v (&m)[2][2], float (&o)[4][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) R3[(16 * (it0 + a) + 4 * lg + r) * KP + 16 * (dt0 + b) + l16] = m[a][b][r];
    kda::lds_barrier();
#pragma unroll
    for (int r = 0; r < 4; ++r) ld4(R3 + (i0 + r) * KP + d0, o[r]);
    kda::lds_barrier();
  };
  to_tiles(mq, aq);
  float dgam[4] = {};   // read before the next barriers (R4 takes dAqk below)
  if (rb == 0)
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) dgam[cc] = R4[d0 + cc] + R4[KD + d0 + cc] + R4[2 * KD + d0 + cc] + R4[3 * KD + d0 + cc];
  to_tiles(mk, akg);
  // Phase 2's global operands, loaded now so that they arrive during the
  // epilogue and dAqk: v (bf16; row u / 16, 8 values from column
  // 8 (u % 16), for u = t, t + 512) and E^T.
  v4u pv[2];
  v4f pet[4];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int u = tid + NTG * k, j = u >> 4, c8 = u & 15;
    pv[k] = j < nv ? *reinterpret_cast<const v4u*>(p.v + ((t0 + j) * p.HV + hv) * KD + 8 * c8) : v4u{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) pet[k] = ldg4(rec + R_ET + 4 * (tid + NTG * k));
  // Epilogue: dq^ = K^-1/2 dQg exp(G); dG = dQg Qg - dKg Kg;
  // dk^ = dKg exp(G_last - G); dG_last partials dKg Kg (+ dgamma gamma).
  {
    float dglp[4];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) dglp[cc] = dgam[cc] * egm[cc];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + r;
      float vq[4], vk[4], vg[4];
      const float qn[4] = {kda::bf16lo(eqn[r].x), kda::bf16hi(eqn[r].x), kda::bf16lo(eqn[r].y), kda::bf16hi(eqn[r].y)};
      const float kn[4] = {kda::bf16lo(ekn[r].x), kda::bf16hi(ekn[r].x), kda::bf16lo(ekn[r].y), kda::bf16hi(ekn[r].y)};
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const float eg = ex2(egv[r][cc]);
        const float el = ex2(egl[cc] - egv[r][cc]);
        const float qg = kScale * qn[cc] * eg;
        const float kg = kn[cc] * el;
        vq[cc] = kScale * aq[r][cc] * eg;
        vg[cc] = aq[r][cc] * qg - akg[r][cc] * kg;
        vk[cc] = akg[r][cc] * el;
        dglp[cc] = fmaf(akg[r][cc], kg, dglp[cc]);
      }
      st4(gdG + i * KD + d0, vg);
      pdk[r] = i < nv ? v4f{vk[0], vk[1], vk[2], vk[3]} : v4f{0.f, 0.f, 0.f, 0.f};
      if (i < nv) {
        st4(gdq + i * rs + d0, vq);
      }
    }
    st4(R3 + rb * KD + d0, dglp);   // [16][128] partials (R3 is free)
  }
  // dAqk (lower triangle incl. the diagonal) into R4, on MFMA.
  {
    f32x4v acc[2] = {f32x4v{0.f, 0.f, 0.f, 0.f}, f32x4v{0.f, 0.f, 0.f, 0.f}};
    tri_mfma(acc, R0, R1, LQ, KD, wave, lg, l16);
    tri_store(R4, LQ, acc, wave, lg, l16, tid);
  }
  kda::lds_barrier();
  if (tid < KD) {
    float sacc = 0.0f;
    for (int r = 0; r < C / 4; ++r) sacc += R3[r * KD + tid];
    sGl[tid] = sacc;
  }
  // ---- phase 2: dA = tril(dVnew v^T + dW E^T), dv = A^T dVnew,
  // dE = A^T dW.  R0 = dW^T [K][C]; R1 = v^T then E^T ([*][C]);
  // R2 = dVnew^T; R3 = dW [C][K].
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) R0[(16 * (dt0 + b) + l16) * LQ + 16 * (it0 + a) + 4 * lg + r] = -mw[a][b][r];
  kda::lds_barrier();   // sGl has read R3's partials
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) R3[(16 * (it0 + a) + 4 * lg + r) * KP + 16 * (dt0 + b) + l16] = -mw[a][b][r];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int u = tid + NTG * k, j = u >> 4, c8 = u & 15;
    const uint32_t w[4] = {pv[k].x, pv[k].y, pv[k].z, pv[k].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      R1[(8 * c8 + 2 * e) * LQ + j] = kda::bf16lo(w[e]);
      R1[(8 * c8 + 2 * e + 1) * LQ + j] = kda::bf16hi(w[e]);
    }
  }
  kda::lds_barrier();
  f32x4v da[2] = {f32x4v{0.f, 0.f, 0.f, 0.f}, f32x4v{0.f, 0.f, 0.f, 0.f}};   // dA's lower tiles, on MFMA
  tri_mfma(da, R2, R1, LQ, KD, wave, lg, l16);
  kda::lds_barrier();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int u = tid + NTG * k, row = u / (C / 4), c4 = u - row * (C / 4);
    sts4(R1 + row * LQ + 4 * c4, pet[k]);
  }
  // The dv / dE operands, loaded during the second half of dA.
  v4f pa[2], ptt[2], pdv[4], pp[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    pa[k] = ldg4(rec + R_A + 4 * (tid + NTG * k));
    ptt[k] = ldg4(rec + R_T + 4 * (tid + NTG * k));
    pp[k] = ldg4(rec + R_P + 4 * (tid + NTG * k));
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) pdv[k] = ldg4(rec + R_DVNT + 4 * (tid + NTG * k));   // dVnew^T [V][C]
  kda::lds_barrier();
  tri_mfma(da, R0, R1, LQ, KD, wave, lg, l16);
  kda::lds_barrier();
  // R0 = A | T ([C][LQ] each); R1 = dA | X; R2 = dVnew [C][K].
  float* sA = R0;
  float* sT = R0 + C * LQ;
  float* sDA = R1;
  float* sX = R1 + C * LQ;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int u = tid + NTG * k, row = u / (C / 4), c4 = u - row * (C / 4);
    sts4(sA + row * LQ + 4 * c4, pa[k]);
    sts4(sT + row * LQ + 4 * c4, ptt[k]);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {   // dVnew [C][K] from its transpose: piece u is row v = u / 16, tokens 4 (u % 16) ..
    const int u = tid + NTG * k, v = u / (C / 4), c4 = u - v * (C / 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) R2[(4 * c4 + e) * KP + v] = pdv[k][e];
  }
  tri_store(sDA, LQ, da, wave, lg, l16, tid);
  kda::lds_barrier();
  {
    // G, k^ (for E = exp(G) k^, formed here as the recompute kernel forms
    // it) and this tile's own dG and dk^ partials, issued before the
    // products.
    v4f xg[4], xdg[4], xdk[4];
    uint2 xk[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = i0 + r;
      xg[r] = ldg4(rec + R_G + j * KD + d0);
      xk[r] = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(rec + R_KN) + j * KD + d0);
      xdg[r] = ldg4(gdG + j * KD + d0);
      xdk[r] = pdk[r];
    }
    float av[4][4] = {}, ae[4][4] = {};
#pragma unroll 4
    for (int i = 0; i < C; ++i) {
      const float4 a = lds4(sA + i * LQ + i0);   // A[i][j] for this tile's rows j
      fma4x4(av, a, lds4(R2 + i * KP + d0), 1.0f);
      fma4x4(ae, a, lds4(R3 + i * KP + d0), 1.0f);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = i0 + r;
      if (j < nv) put4(p.dv, ((t0 + j) * p.HV + hv) * KD + d0, av[r], p.obf);
      float vg[4], vk[4];
      const float kf[4] = {kda::bf16lo(xk[r].x), kda::bf16hi(xk[r].x), kda::bf16lo(xk[r].y), kda::bf16hi(xk[r].y)};
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const float eg = ex2(xg[r][cc]);
        vg[cc] = fmaf(ae[r][cc], eg * kf[cc], xdg[r][cc]);
        vk[cc] = fmaf(ae[r][cc], eg, xdk[r][cc]);
      }
      st4(gdG + j * KD + d0, vg);
      pdk[r] = j < nv ? v4f{vk[0], vk[1], vk[2], vk[3]} : v4f{0.f, 0.f, 0.f, 0.f};
    }
  }
  // ---- dbeta and dL: dbeta_j += sum_i dA_ij T_ij; dT = dA diag(beta);
  // X = dT T^T; dL = -tril_strict(T^T X) (into sDA); dbeta_i += sum_j dL_ij P_ij.
  // Eight lanes per column (rows p, p + 8, ...), summed across the lanes by DPP.
  static_assert(NTG == 8 * C, "one 8-lane group per row or column of the chunk");
  {
    const int j = tid >> 3, p = tid & 7;
    float acc = 0.0f;
#pragma unroll
    for (int m = 0; m < C / 8; ++m) {
      const int i = p + 8 * m;
      if (i >= j) acc = fmaf(sDA[i * LQ + j], sT[i * LQ + j], acc);
    }
    acc += __uint_as_float(kda::dpp32<kda::kDppXor1>(__float_as_uint(acc)));
    acc += __uint_as_float(kda::dpp32<kda::kDppXor2>(__float_as_uint(acc)));
    acc += __uint_as_float(kda::dpp32<kda::kDppHalfMirror>(__float_as_uint(acc)));
    if (p == 0) sDB[j] += acc;
  }
  kda::lds_barrier();
  for (int t = tid; t < C * C; t += NTG) {
    const int i = t / C, j = t - i * C;
    sDA[i * LQ + j] *= sB[j];
  }
  kda::lds_barrier();
  // Phase 3's operands (G, k^, q^), loaded while dbeta, X and dL run.
  v4f pg3[4];
  uint2 pk3[4], pq3[4];   // bf16 k^ and q^, four per piece
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    pg3[k] = ldg4(rec + R_G + 4 * (tid + NTG * k));
    pk3[k] = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(rec + R_KN) + 4 * (tid + NTG * k));
    pq3[k] = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(rec + R_QN) + 4 * (tid + NTG * k));
  }
  // dT^T and T^T (R2 and R3 are free: dv and dE are done) and P.
  float* sDTT = R2;
  float* sTT = R2 + C * LQ;
  float* sP = R3;
  for (int t = tid; t < C * C; t += NTG) {
    const int i = t / C, j = t - i * C;
    sDTT[j * LQ + i] = sDA[i * LQ + j];
    sTT[j * LQ + i] = sT[i * LQ + j];
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int u = tid + NTG * k, row = u / (C / 4), c4 = u - row * (C / 4);
    sts4(sP + row * LQ + 4 * c4, pp[k]);
  }
  kda::lds_barrier();
  // X = dT T^T on MFMA: X[i][m] = sum_j dT[i][j] T[m][j] (j <= min(i, m),
  // so tile (I, J) stops at k = 16 (min(I, J) + 1)); wave w takes tiles w
  // and w + 8 of the 4x4 grid.
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = wave + 8 * h, I = t >> 2, J = t & 3;
    const f32x4v acc = tile_mfma(f32x4v{0.f, 0.f, 0.f, 0.f}, sDTT, sTT, LQ, I, J, 0, 16 * (min(I, J) + 1), lg, l16);
#pragma unroll
    for (int r = 0; r < 4; ++r) sX[(16 * I + 4 * lg + r) * LQ + 16 * J + l16] = acc[r];
  }
  kda::lds_barrier();
  // dL = -tril_strict(T^T X) on MFMA: dL[a][b] = -sum_{i >= a} T[i][a] X[i][b]
  // (T stored row-major is T^T stored transposed), lower tiles into sDA;
  // the tiles above hold dT's zeros already.
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = wave + 8 * h;
    if (t >= 10) break;
    int I, J;
    tri_tile(t, I, J);
    const f32x4v acc = tile_mfma(f32x4v{0.f, 0.f, 0.f, 0.f}, sT, sX, LQ, I, J, 16 * I, C, lg, l16);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int a = 16 * I + 4 * lg + r, b = 16 * J + l16;
      sDA[a * LQ + b] = (b < a) ? -acc[r] : 0.0f;
    }
  }
  kda::lds_barrier();
  {
    const int i = tid >> 3, p = tid & 7;
    float acc = 0.0f;
#pragma unroll
    for (int m = 0; m < C / 8; ++m) {
      const int j = p + 8 * m;
      if (j < i) acc = fmaf(sDA[i * LQ + j], sP[i * LQ + j], acc);
    }
    acc += __uint_as_float(kda::dpp32<kda::kDppXor1>(__float_as_uint(acc)));
    acc += __uint_as_float(kda::dpp32<kda::kDppXor2>(__float_as_uint(acc)));
    acc += __uint_as_float(kda::dpp32<kda::kDppHalfMirror>(__float_as_uint(acc)));
    if (p == 0) sDB[i] += acc;
  }
  kda::lds_barrier();   // R2 and R3 are reloaded below
  // ---- phase 3: gated sums.  R0 = G, R2 = k^, R3 = q^ ([C][K]); dL in
  // R1 (sDA), dAqk in R4.
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int u = tid + NTG * k, row = u / (KD / 4), c4 = u - row * (KD / 4);
    sts4(R0 + row * KP + 4 * c4, pg3[k]);
    sts4(R2 + row * KP + 4 * c4, v4f{kda::bf16lo(pk3[k].x), kda::bf16hi(pk3[k].x), kda::bf16lo(pk3[k].y), kda::bf16hi(pk3[k].y)});
    sts4(R3 + row * KP + 4 * c4, v4f{kda::bf16lo(pq3[k].x), kda::bf16hi(pq3[k].x), kda::bf16lo(pq3[k].y), kda::bf16hi(pq3[k].y)});
  }
  kda::lds_barrier();
  float dgt[4][4];   // this tile's final dG (written to LDS once all of phase 3 is done)
  float fk[4][4];    // this tile's final dk^
  {
    float gi[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) ld4(R0 + (i0 + r) * KP + d0, gi[r]);
    // Row forms: j <= i over this tile's rows i.  Below the tile's first
    // row i0 the factor splits around it, exp(G_i - G_j) =
    // exp(G_i - G_i0) exp(G_i0 - G_j), both <= 1.  The first part (with
    // beta_i and the scale) does not depend on j, so the loop sums the
    // second part only and the first is applied once after it; the tile's
    // own 4x4 diagonal block is formed directly (j <= i only).
    {
      float rk[4][4] = {}, rq[4][4] = {};
      for (int j4 = 0; j4 < i0; j4 += 4) {
        float dl[4][4], aq[4][4];   // [row r][column j4 + jj]
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          ld4(sDA + (i0 + r) * LQ + j4, dl[r]);
          ld4(R4 + (i0 + r) * LQ + j4, aq[r]);
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          float gj[4], kj[4], fc[4];
          ld4(R0 + (j4 + jj) * KP + d0, gj);
          ld4(R2 + (j4 + jj) * KP + d0, kj);
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) fc[cc] = ex2(gi[0][cc] - gj[cc]) * kj[cc];
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
              rk[r][cc] = fmaf(dl[r][jj], fc[cc], rk[r][cc]);
              rq[r][cc] = fmaf(aq[r][jj], fc[cc], rq[r][cc]);
            }
        }
      }
      // This tile's dG, dq^ and dk^ so far (phase 2 stored their last
      // parts), all four rows loaded before any is stored.
      v4f zdg[4], zdq[4], zdk[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + r;
        zdg[r] = ldg4(gdG + i * KD + d0);
        zdq[r] = i < nv ? ldg4(gdq + i * rs + d0) : v4f{0.f, 0.f, 0.f, 0.f};
        zdk[r] = pdk[r];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float bi = sB[i0 + r];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const float f = ex2(gi[r][cc] - gi[0][cc]);
          rk[r][cc] *= bi * f;
          rq[r][cc] *= kScale * f;
        }
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = i0 + jj;
        float gj[4], kj[4];
        ld4(R0 + j * KP + d0, gj);
        ld4(R2 + j * KP + d0, kj);
#pragma unroll
        for (int r = jj; r < 4; ++r) {
          const int i = i0 + r;
          const float mk = sB[i] * sDA[i * LQ + j];
          const float mq = kScale * R4[i * LQ + j];
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) {
            const float e = ex2(gi[r][cc] - gj[cc]) * kj[cc];
            rk[r][cc] = fmaf(mk, e, rk[r][cc]);
            rq[r][cc] = fmaf(mq, e, rq[r][cc]);
          }
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + r;
        float ki[4], qi[4], vq[4];
        ld4(R2 + i * KP + d0, ki);
        ld4(R3 + i * KP + d0, qi);
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          dgt[r][cc] = zdg[r][cc] + ki[cc] * rk[r][cc] + qi[cc] * rq[r][cc];
          vq[cc] = zdq[r][cc] + rq[r][cc];
          zdk[r][cc] += rk[r][cc];
        }
        if (i < nv) st4(gdq + i * rs + d0, vq);
        pdk[r] = i < nv ? zdk[r] : v4f{0.f, 0.f, 0.f, 0.f};
      }
    }
    // Column forms: i >= j over this tile's rows j (as the column index).
    // Past the tile's last row i0 + 3 the factor splits around it, both
    // parts <= 1; the part exp(G_{i0+3} - G_j) does not depend on i and is
    // applied once after the loop (the scale of the q form with it).  The
    // diagonal block is formed directly (i >= j only).
    {
      float ck[4][4] = {}, cq[4][4] = {};
#pragma unroll 2
      for (int i = i0 + 4; i < C; ++i) {
        float gr[4], kr[4], qr[4], dl[4], aqv[4];
        ld4(R0 + i * KP + d0, gr);
        ld4(R2 + i * KP + d0, kr);
        ld4(R3 + i * KP + d0, qr);
        ld4(sDA + i * LQ + i0, dl);
        ld4(R4 + i * LQ + i0, aqv);
        const float bi = sB[i];
        float kf[4], qf[4];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const float fi = ex2(gr[cc] - gi[3][cc]);
          kf[cc] = bi * kr[cc] * fi;
          qf[cc] = qr[cc] * fi;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) {
            ck[r][cc] = fmaf(dl[r], kf[cc], ck[r][cc]);
            cq[r][cc] = fmaf(aqv[r], qf[cc], cq[r][cc]);
          }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const float f = ex2(gi[3][cc] - gi[r][cc]);
          ck[r][cc] *= f;
          cq[r][cc] *= kScale * f;
        }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int i = i0 + ii;
        float gr[4], kr[4], qr[4];
        ld4(R0 + i * KP + d0, gr);
        ld4(R2 + i * KP + d0, kr);
        ld4(R3 + i * KP + d0, qr);
        const float bi = sB[i];
#pragma unroll
        for (int r = 0; r <= ii; ++r) {
          const float mk = bi * sDA[i * LQ + i0 + r];
          const float mq = kScale * R4[i * LQ + i0 + r];
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) {
            const float e = ex2(gr[cc] - gi[r][cc]);
            ck[r][cc] = fmaf(mk, kr[cc] * e, ck[r][cc]);
            cq[r][cc] = fmaf(mq, qr[cc] * e, cq[r][cc]);
          }
        }
      }
      v4f yk[4];   // dk^ as the row forms left it, all four rows loaded first
#pragma unroll
      for (int r = 0; r < 4; ++r) yk[r] = pdk[r];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + r;
        float ki[4];
        ld4(R2 + i * KP + d0, ki);
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) dgt[r][cc] -= ki[cc] * (ck[r][cc] + cq[r][cc]);
        if (i == C - 1)
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) dgt[r][cc] += sGl[d0 + cc];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) fk[r][cc] = yk[r][cc] + ck[r][cc] + cq[r][cc];
        if (i < nv && !fused) st4(gdk + i * rs + d0, fk[r]);
      }
    }
  }
  // ---- outputs: dg as the reverse prefix of dG over the chunk's rows
  // (dG_last was added to the last row), in four 16-row blocks per column:
  // suffix sums within each block, then the totals of the later blocks.
  kda::lds_barrier();
  // With one value head per Q/K head the normalisation's backward runs here
  // too (below): this tile's raw q and k and its final dq^, loaded now.
  uint2 xq[4], xk[4];
  v4f fq[4];
  if (fused) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + r;
      const bool ok = i < nv;
      const int64_t xo = ((t0 + i) * p.H + hv) * KD + d0;
      xq[r] = ok ? *reinterpret_cast<const uint2*>(p.q + xo) : make_uint2(0u, 0u);
      xk[r] = ok ? *reinterpret_cast<const uint2*>(p.k + xo) : make_uint2(0u, 0u);
      fq[r] = ok ? ldg4(gdq + i * rs + d0) : v4f{0.f, 0.f, 0.f, 0.f};
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) st4(R0 + (i0 + r) * KP + d0, dgt[r]);
  kda::lds_barrier();
  {
    const int d = tid & (KD - 1), blk = tid >> 7;
    float acc = 0.0f;
#pragma unroll
    for (int r = 15; r >= 0; --r) {
      acc += R0[(16 * blk + r) * KP + d];
      R0[(16 * blk + r) * KP + d] = acc;
    }
    kda::lds_barrier();
    float later = 0.0f;
    for (int b = blk + 1; b < C / 16; ++b) later += R0[16 * b * KP + d];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 16 * blk + r;
      if (i < nv) p.dg[((t0 + i) * p.HV + hv) * KD + d] = R0[i * KP + d] + later;
    }
  }
  if (tid < nv) put1(p.dbeta, (t0 + tid) * p.HV + hv, sDB[tid], p.obf);
  // Normalisation backward (one value head per Q/K head): for x the raw row,
  // n = sqrt(sum x^2 + 1e-6), dx = dy / n - x (x . dy) / n^3; the sums over
  // a row's 128 channels run across the 32 lanes that hold it.
  if (fused) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float xqv[4] = {kda::bf16lo(xq[r].x), kda::bf16hi(xq[r].x), kda::bf16lo(xq[r].y), kda::bf16hi(xq[r].y)};
      const float xkv[4] = {kda::bf16lo(xk[r].x), kda::bf16hi(xk[r].x), kda::bf16lo(xk[r].y), kda::bf16hi(xk[r].y)};
      float sq = 0.f, dq_ = 0.f, sk = 0.f, dk_ = 0.f;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        sq = fmaf(xqv[cc], xqv[cc], sq);
        dq_ = fmaf(xqv[cc], fq[r][cc], dq_);
        sk = fmaf(xkv[cc], xkv[cc], sk);
        dk_ = fmaf(xkv[cc], fk[r][cc], dk_);
      }
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) {
        sq += __shfl_xor(sq, off, 32);
        dq_ += __shfl_xor(dq_, off, 32);
        sk += __shfl_xor(sk, off, 32);
        dk_ += __shfl_xor(dk_, off, 32);
      }
      const int i = i0 + r;
      if (i < nv) {
        const float iq = 1.0f / sqrtf(sq + 1e-6f), ik = 1.0f / sqrtf(sk + 1e-6f);
        const float cq3 = dq_ * iq * iq * iq, ck3 = dk_ * ik * ik * ik;
        float oq[4], ok[4];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          oq[cc] = fq[r][cc] * iq - xqv[cc] * cq3;
          ok[cc] = fk[r][cc] * ik - xkv[cc] * ck3;
        }
        const int64_t o = ((t0 + i) * p.H + hv) * KD + d0;
        put4(p.dq, o, oq, p.obf);
        put4(p.dk, o, ok, p.obf);
      }
    }
  }
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
  void* out = isk ? p.dk : p.dq;
#pragma unroll
  for (int e = 0; e < 2; ++e) put1(out, r * KD + lane + 64 * e, gv[e] * inv - xv[e] * c3, p.obf);
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
                                  const void* d_out, const float* d_final_state, void* dq, void* dk, void* dv,
                                  float* dg, void* dbeta, float* d_initial_state, int32_t grad_dtype,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  // HV <= 65535: value heads are a launch-grid dimension.
  if (B < 1 || T < 0 || H < 1 || HV < 1 || HV > 65535 || HV % H != 0) return KDA_ERR_SHAPE;
  if (Kd != KD || Vd != KD) return KDA_ERR_UNSUPPORTED;
  if (grad_dtype != KDA_GRAD_FLOAT32 && grad_dtype != KDA_GRAD_INPUT_DTYPE) return KDA_ERR_UNSUPPORTED;
  if (cu_seqlens && (B != 1 || num_seqs < 1)) return KDA_ERR_SHAPE;
  const int64_t nseq = cu_seqlens ? num_seqs : B;
  const int64_t tokens = int64_t(B) * T;
  if (tokens > 0 && (!q || !k || !v || !g || !beta || !d_out || !dq || !dk || !dv || !dg || !dbeta))
    return KDA_ERR_NULL;
  if (!kda::aligned16(q) || !kda::aligned16(k) || !kda::aligned16(v) || !kda::aligned16(g) ||
      !kda::aligned16(d_out) || !kda::aligned16(dq) || !kda::aligned16(dk) || !kda::aligned16(dv) ||
      !kda::aligned16(dg) || !kda::aligned16(workspace) || !kda::aligned16(initial_state) ||
      !kda::aligned16(d_final_state) || !kda::aligned16(d_initial_state))
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
  p.obf = grad_dtype == KDA_GRAD_INPUT_DTYPE;

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
  hipLaunchKernelGGL(bwd_prep_kernel, chunks, dim3(NTP), PREP_LDS, s, p);
  int st = kda::launch_status();
  if (st != KDA_OK) return st;
  hipLaunchKernelGGL(bwd_carry_fwd_kernel, carries, dim3(NTC), FWD_LDS, s, p);
  st = kda::launch_status();
  if (st != KDA_OK) return st;
  hipLaunchKernelGGL(bwd_carry_rev_kernel, carries, dim3(NTC), REV_LDS, s, p);
  st = kda::launch_status();
  if (st != KDA_OK) return st;
  if (tokens == 0) return KDA_OK;
  hipLaunchKernelGGL(bwd_grad_kernel, chunks, dim3(NTG), GRAD_LDS, s, p);
  st = kda::launch_status();
  if (st != KDA_OK) return st;
  if (H == HV) return KDA_OK;   // the gradient kernel ran the normalisation backward
  const int64_t rows = 2 * tokens * H;
  hipLaunchKernelGGL(bwd_norm_kernel, dim3(unsigned((rows + NTB / 64 - 1) / (NTB / 64))), dim3(NTB), 0, s, p);
  return kda::launch_status();
}
