// KDA chunked prefill (export kda_chunk_prefill).
//
// Page "KDA Chunk Prefill on Ascend A3": section "Function and tensor
// contract" (shapes, GQA head mapping) and section "Mathematical definition"
// (Q/K L2 normalisation; the chunk construction G, L, A = solve(I+L,
// diag(beta)), W, U, Qg, Kg, Aqk; the carry Vnew = U - W S, O = Qg S + Aqk
// Vnew, S = exp(G_last) S + Kg^T Vnew; chunk size 64 with a zero-padded last
// chunk).
//
// Design (one fused kernel, no workspace):
//   * one workgroup per (sequence, value head, V-tile); the V-tile is 64 or
//     128 columns of the 128-column state, because the state's columns
//     evolve independently (each column of S only ever meets the same column
//     of v).  Each wave owns 16 columns of the tile and keeps that 128x16
//     slice of S in registers as float32 for the whole sequence.
//   * per 64-token chunk, all waves build the chunk-local quantities in LDS:
//     normalised q and k (bit-exact routine shared with kda_qk_l2norm), the
//     gate prefix G (kept in log2 units), the gated L and Aqk on MFMA, the
//     unit-lower-triangular inverse by blocked forward substitution in
//     float32, A, W = A (exp(G) k), Qg, Kg and exp(G_last).
//   * then each wave runs the carry for its columns on MFMA: U = A v and
//     Vnew = U - W S accumulate in float32 (U is never rounded), O = Qg S +
//     Aqk Vnew, S = exp(G_last) S + Kg^T Vnew.
//
// Precision: every MFMA operand is fp16 with float32 accumulation, and the
// state is carried in float32.  fp16's 11-bit significand keeps the final
// state within a few 1e-4 (relative Frobenius) of the float64 recurrence
// even when beta = 1 and the gates barely decay, where bf16 operands drift
// past 1e-3.  The operands are bounded in magnitude (|A| <= 1, decay factors
// <= 1, normalised q and k), except v, the state and the split decay factors
// of diagonal blocks: v and the state must stay below 2^14 in magnitude, and
// a diagonal block whose split factors exceed 2^14 (gates below about -1.2
// per token) is computed with bf16 operands instead.
//
// Overflow-safe decay factors.  exp(G_i - G_j) for j <= i is <= 1, but it is
// needed inside dot products over the channel d, so it is split into a row
// factor and a column factor around a reference token r:
//   exp(G_i - G_j) = exp(G_i - G_r) * exp(G_r - G_j).
// For a 16x16 block below the diagonal, r is the first token of the row
// block, so both factors are <= 1.  For a diagonal block, r is the block's
// middle token, so each factor is at most exp of the decay accumulated over
// 8 tokens; if that exceeds 2^120 for any channel the block is computed
// pair by pair instead (exact, slow, only for extreme gates).  exp(-G) over a
// whole chunk is never formed.
#include <atomic>

#include "kda_device.h"
#include "kda_host.h"

namespace {

using namespace kda;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int C = 64;            // chunk length
constexpr int KD = 128;          // key width == value width
constexpr float LOG2E = 1.4426950408889634f;
constexpr float SCALE = 0.08838834764831845f;   // 128^-1/2
constexpr float SAFE_EXP2 = 120.0f;             // largest split-factor exponent (base 2)
constexpr float F16_EXP2 = 14.0f;               // largest split-factor exponent for fp16 operands

// LDS row strides (elements); the padding breaks power-of-two bank strides.
constexpr int QS = 136;          // bf16 [64][128] arrays
constexpr int GS = 132;          // fp32 G [64][128]
constexpr int LS = 68;           // fp32 [64][64] arrays
constexpr int AS = 72;           // 16-bit [*][64] arrays

// LDS map (bytes).  U1 holds L and T during the solve and W and E^T after.
constexpr int OFF_Q = 0;                                  // bf16 q^ -> Qg   [64][QS]
constexpr int OFF_K = OFF_Q + C * QS * 2;                 // bf16 k^         [64][QS]
constexpr int OFF_G = OFF_K + C * QS * 2;                 // fp32 G (log2)   [64][GS]
constexpr int OFF_U1 = OFF_G + C * GS * 4;
constexpr int OFF_L = OFF_U1;                             // fp32 L          [64][LS]
constexpr int OFF_T = OFF_U1 + C * LS * 4;                // fp32 (I+L)^-1   [64][LS]
constexpr int OFF_W = OFF_U1;                             // bf16 -W         [64][QS]
constexpr int OFF_ET = OFF_U1 + C * QS * 2;               // bf16 (e^G k)^T  [128][AS]
constexpr int U1_BYTES = (2 * C * LS * 4 > C * QS * 2 + KD * AS * 2) ? 2 * C * LS * 4
                                                                     : C * QS * 2 + KD * AS * 2;
constexpr int OFF_AQK = OFF_U1 + U1_BYTES;                // bf16 Aqk        [64][AS]
constexpr int OFF_A = OFF_AQK + C * AS * 2;               // bf16 A [64][AS]; fp32 solve scratch
constexpr int OFF_KGT = OFF_A + C * AS * 2;               // fp16 Kg^T       [128][AS]
constexpr int OFF_VT = OFF_KGT + KD * AS * 2;             // bf16 v^T        [VT][AS]

template <int VT>
struct Lds {
  static constexpr int OFF_BETA = OFF_VT + VT * AS * 2;   // fp32 [64]
  static constexpr int OFF_GAM = OFF_BETA + C * 4;        // fp32 [128]
  static constexpr int BYTES = OFF_GAM + KD * 4;
};
static_assert(Lds<128>::BYTES <= 160 * 1024, "LDS budget");
static_assert(C * AS * 2 >= 3 * 256 * 4, "solve scratch fits in the A region");

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* g;
  const uint16_t* beta;
  const float* s0;
  const int32_t* cu;
  uint16_t* o;
  float* sfin;
  int B, T, H, HV, N;
};

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f16x8 lds_f16x8(const uint16_t* p) {
  return *reinterpret_cast<const f16x8*>(p);
}
__device__ __forceinline__ f16x8 lds_f16_2x4(const uint16_t* p0, const uint16_t* p1) {
  uint2 a = *reinterpret_cast<const uint2*>(p0);
  uint2 b = *reinterpret_cast<const uint2*>(p1);
  uint4 u = make_uint4(a.x, a.y, b.x, b.y);
  return __builtin_bit_cast(f16x8, u);
}
__device__ __forceinline__ uint16_t f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

template <int VT>
__global__ __launch_bounds__(VT * 4) void prefill_kernel(Params p) {
  constexpr int NW = VT / 16;          // waves; wave w owns tile columns 16w..16w+15
  constexpr int NT = NW * 64;
  constexpr int NV = KD / VT;          // V-tiles per head
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* sQ = reinterpret_cast<uint16_t*>(smem + OFF_Q);
  uint16_t* sK = reinterpret_cast<uint16_t*>(smem + OFF_K);
  float* sG = reinterpret_cast<float*>(smem + OFF_G);
  float* sL = reinterpret_cast<float*>(smem + OFF_L);
  float* sT = reinterpret_cast<float*>(smem + OFF_T);
  uint16_t* sW = reinterpret_cast<uint16_t*>(smem + OFF_W);
  uint16_t* sET = reinterpret_cast<uint16_t*>(smem + OFF_ET);
  uint16_t* sAqk = reinterpret_cast<uint16_t*>(smem + OFF_AQK);
  uint16_t* sA = reinterpret_cast<uint16_t*>(smem + OFF_A);
  float* sP = reinterpret_cast<float*>(smem + OFF_A);      // solve scratch [3][16][16]
  uint16_t* sKgT = reinterpret_cast<uint16_t*>(smem + OFF_KGT);
  uint16_t* sVT = reinterpret_cast<uint16_t*>(smem + OFF_VT);
  float* sBeta = reinterpret_cast<float*>(smem + Lds<VT>::OFF_BETA);
  float* sGam = reinterpret_cast<float*>(smem + Lds<VT>::OFF_GAM);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int gq = lane >> 4;

  // Workgroup -> (unit = sequence*HV + head, V-tile); the NV tiles of a unit
  // get ids congruent mod 8 so they share an XCD (and its L2).
  const int id = blockIdx.x;
  const int grp = id / (8 * NV);
  const int rem = id % (8 * NV);
  const int vt = rem / 8;
  const int unit = grp * 8 + (rem % 8);
  if (unit >= p.N * p.HV) return;
  const int n = unit / p.HV;
  const int hv = unit % p.HV;
  const int hq = hv / (p.HV / p.H);

  int64_t tok0;   // row index (into the [B*T] token axis) of the sequence's first token
  int len;
  if (p.cu) {
    tok0 = p.cu[n];
    len = p.cu[n + 1] - p.cu[n];
  } else {
    tok0 = int64_t(n) * p.T;
    len = p.T;
  }

  const int col = vt * VT + wave * 16 + l16;     // this lane's state / output column
  f32x4 S[8];                                    // rows 16rt + 4gq + r of column `col`
  {
    const float* s0 = p.s0 ? p.s0 + (int64_t(n) * p.HV + hv) * KD * KD : nullptr;
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) S[rt][r] = s0 ? s0[(16 * rt + 4 * gq + r) * KD + col] : 0.f;
  }

  for (int c0 = 0; c0 < len; c0 += C) {
    const int nvalid = min(C, len - c0);
    const int64_t trow = tok0 + c0;              // token row of chunk position 0

    // ---------------------------------------------------------- phase 1: loads
    // q^ and k^: 128 rows, one 16-lane group per row, bit-exact normalisation.
    for (int r = tid >> 4; r < 2 * C; r += NT / 16) {
      const int i = r & (C - 1);
      const bool isk = r >= C;
      uint4 x = make_uint4(0u, 0u, 0u, 0u);
      if (i < nvalid) {
        const uint16_t* src = (isk ? p.k : p.q) + ((trow + i) * p.H + hq) * KD + 8 * l16;
        x = *reinterpret_cast<const uint4*>(src);
      }
      uint4 y = l2norm_row16(x);
      *reinterpret_cast<uint4*>((isk ? sK : sQ) + i * QS + 8 * l16) = y;
    }
    // g (scaled to log2 units), beta, v tile (transposed).
    for (int e = tid; e < C * (KD / 4); e += NT) {
      const int i = e / (KD / 4);
      const int c4 = e % (KD / 4);
      float4 gv = make_float4(0.f, 0.f, 0.f, 0.f);
      if (i < nvalid) gv = *reinterpret_cast<const float4*>(p.g + ((trow + i) * p.HV + hv) * KD + 4 * c4);
      float* d = sG + i * GS + 4 * c4;
      d[0] = gv.x * LOG2E;
      d[1] = gv.y * LOG2E;
      d[2] = gv.z * LOG2E;
      d[3] = gv.w * LOG2E;
    }
    if (tid < C) sBeta[tid] = tid < nvalid ? bf16f(p.beta[(trow + tid) * p.HV + hv]) : 0.f;
    for (int e = tid; e < C * (VT / 8); e += NT) {
      const int i = e / (VT / 8);
      const int c8 = e % (VT / 8);
      uint4 x = make_uint4(0u, 0u, 0u, 0u);
      if (i < nvalid)
        x = *reinterpret_cast<const uint4*>(p.v + ((trow + i) * p.HV + hv) * KD + vt * VT + 8 * c8);
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        sVT[(8 * c8 + 2 * q2) * AS + i] = f16_bits(bf16lo(w[q2]));
        sVT[(8 * c8 + 2 * q2 + 1) * AS + i] = f16_bits(bf16hi(w[q2]));
      }
    }
    __syncthreads();
    // G = inclusive prefix over the chunk, per channel (padding has g = 0).
    if (tid < KD) {
      float run = 0.f;
      for (int i = 0; i < C; ++i) {
        run += sG[i * GS + tid];
        sG[i * GS + tid] = run;
      }
    }
    __syncthreads();

    // ---------------------------------------------------------- phase 2: L, Aqk
    for (int pb = wave; pb < 16; pb += NW) {
      const int I = pb >> 2;
      const int J = pb & 3;
      if (J > I) {   // strictly upper blocks of Aqk are zero
#pragma unroll
        for (int r = 0; r < 4; ++r) sAqk[(16 * I + 4 * gq + r) * AS + 16 * J + l16] = 0;
        continue;
      }
      const int ref = (J < I) ? 16 * I : 16 * I + 8;
      const int i = 16 * I + l16;     // operand row (A side)
      const int j = 16 * J + l16;     // operand row (B side)
      // Largest split-factor exponent this lane will form (<= 0 below the diagonal).
      float emax = 0.f;
      if (J == I) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int ch = 32 * s + 8 * gq + e;
            const float gr = sG[ref * GS + ch];
            emax = fmaxf(emax, fmaxf(sG[i * GS + ch] - gr, gr - sG[j * GS + ch]));
          }
      }
      f32x4 accL = {0.f, 0.f, 0.f, 0.f};
      f32x4 accQ = {0.f, 0.f, 0.f, 0.f};
      if (!__any(emax > F16_EXP2)) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int ch0 = 32 * s + 8 * gq;
          f16x8 kr, qr, kc;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int ch = ch0 + e;
            const float gr = sG[ref * GS + ch];
            const float fr = ex2(sG[i * GS + ch] - gr);
            const float fc = ex2(gr - sG[j * GS + ch]);
            kr[e] = (_Float16)(bf16f(sK[i * QS + ch]) * fr);
            qr[e] = (_Float16)(bf16f(sQ[i * QS + ch]) * fr);
            kc[e] = (_Float16)(bf16f(sK[j * QS + ch]) * fc);
          }
          accL = __builtin_amdgcn_mfma_f32_16x16x32_f16(kr, kc, accL, 0, 0, 0);
          accQ = __builtin_amdgcn_mfma_f32_16x16x32_f16(qr, kc, accQ, 0, 0, 0);
        }
      } else {
        // Steep decay inside a diagonal block: bf16 operands keep the range.
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int ch0 = 32 * s + 8 * gq;
          bf16x8 kr, qr, kc;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int ch = ch0 + e;
            const float gr = sG[ref * GS + ch];
            const float fr = ex2(sG[i * GS + ch] - gr);
            const float fc = ex2(gr - sG[j * GS + ch]);
            kr[e] = (__bf16)(bf16f(sK[i * QS + ch]) * fr);
            qr[e] = (__bf16)(bf16f(sQ[i * QS + ch]) * fr);
            kc[e] = (__bf16)(bf16f(sK[j * QS + ch]) * fc);
          }
          accL = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr, kc, accL, 0, 0, 0);
          accQ = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qr, kc, accQ, 0, 0, 0);
        }
      }
      const int jc = 16 * J + l16;    // result column
      if (__any(emax > SAFE_EXP2)) {
        // Extreme decay inside a diagonal block: evaluate each pair directly.
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ir = 16 * I + 4 * gq + r;
          float aL = 0.f, aQ = 0.f;
          if (jc <= ir) {
            for (int ch = 0; ch < KD; ++ch) {
              const float f = ex2(sG[ir * GS + ch] - sG[jc * GS + ch]);
              const float kj = bf16f(sK[jc * QS + ch]) * f;
              aL = fmaf(bf16f(sK[ir * QS + ch]), kj, aL);
              aQ = fmaf(bf16f(sQ[ir * QS + ch]), kj, aQ);
            }
          }
          accL[r] = aL;
          accQ[r] = aQ;
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ir = 16 * I + 4 * gq + r;
        sL[ir * LS + jc] = (jc < ir) ? sBeta[ir] * accL[r] : 0.f;
        const float aq = (jc <= ir) ? SCALE * accQ[r] : 0.f;
        sAqk[ir * AS + jc] = f16_bits(aq);
      }
    }
    __syncthreads();

    // ---------------------------------------------------------- phase 3: solve
    // T = (I + L)^-1, unit lower triangular.  Diagonal 16x16 blocks by forward
    // substitution, one lane per (block, column).
    if (wave == 0) {
      const int blk = lane >> 4;
      const int cc = lane & 15;
      float x[16];
#pragma unroll
      for (int ii = 0; ii < 16; ++ii) {
        float s = 0.f;
#pragma unroll
        for (int m = 0; m < ii; ++m) s = fmaf(sL[(16 * blk + ii) * LS + 16 * blk + m], x[m], s);
        x[ii] = (ii == cc) ? 1.f : (ii > cc ? -s : 0.f);
      }
#pragma unroll
      for (int ii = 0; ii < 16; ++ii) sT[(16 * blk + ii) * LS + 16 * blk + cc] = x[ii];
    }
    __syncthreads();
    // Off-diagonal blocks, one block row at a time:
    //   T_IJ = -T_II * sum_{M=J}^{I-1} L_IM T_MJ.
    for (int I = 1; I < 4; ++I) {
      for (int e = tid; e < I * 256; e += NT) {
        const int J = e >> 8;
        const int ii = (e >> 4) & 15;
        const int jj = e & 15;
        float s = 0.f;
        for (int m = 16 * J; m < 16 * I; ++m) s = fmaf(sL[(16 * I + ii) * LS + m], sT[m * LS + 16 * J + jj], s);
        sP[J * 256 + ii * 16 + jj] = s;
      }
      __syncthreads();
      for (int e = tid; e < I * 256; e += NT) {
        const int J = e >> 8;
        const int ii = (e >> 4) & 15;
        const int jj = e & 15;
        float s = 0.f;
#pragma unroll
        for (int m = 0; m < 16; ++m) s = fmaf(sT[(16 * I + ii) * LS + 16 * I + m], sP[J * 256 + m * 16 + jj], s);
        sT[(16 * I + ii) * LS + 16 * J + jj] = -s;
      }
      __syncthreads();
    }
    // A = T diag(beta), lower triangular, as fp16.
    for (int e = tid; e < C * C; e += NT) {
      const int ii = e >> 6;
      const int jj = e & 63;
      const float a = (jj <= ii) ? sT[ii * LS + jj] * sBeta[jj] : 0.f;
      sA[ii * AS + jj] = f16_bits(a);
    }
    __syncthreads();

    // ---------------------------------------------------------- phase 4: W, Qg, Kg
    if (tid < KD) sGam[tid] = ex2(sG[(C - 1) * GS + tid]);
    for (int e = tid; e < C * KD; e += NT) {
      const int jj = e >> 7;
      const int c = e & (KD - 1);
      const float gj = sG[jj * GS + c];
      const float glast = sG[(C - 1) * GS + c];
      const float kk = bf16f(sK[jj * QS + c]);
      const float eg = ex2(gj);
      sET[c * AS + jj] = f16_bits(kk * eg);
      sKgT[c * AS + jj] = f16_bits(kk * ex2(glast - gj));
      const float qq = bf16f(sQ[jj * QS + c]);
      sQ[jj * QS + c] = f16_bits(SCALE * qq * eg);
    }
    __syncthreads();
    // W = A (e^G k): 4 x 8 output tiles, A is lower triangular.
    for (int pt = wave; pt < 32; pt += NW) {
      const int mt = pt >> 3;
      const int nt = pt & 7;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int s = 0; s <= (mt >> 1); ++s) {
        const f16x8 a = lds_f16x8(sA + (16 * mt + l16) * AS + 32 * s + 8 * gq);
        const f16x8 b = lds_f16x8(sET + (16 * nt + l16) * AS + 32 * s + 8 * gq);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) sW[(16 * mt + 4 * gq + r) * QS + 16 * nt + l16] = f16_bits(-acc[r]);
    }
    __syncthreads();

    // ---------------------------------------------------------- phase 5: carry
    // Contraction orders: for products with S the channel index of k-slot
    // (gq, e) is 32s + 4gq + e (e < 4) or 32s + 16 + 4gq + (e - 4), which is
    // exactly where the float32 S accumulator already holds it; products with
    // Vnew use the same permutation over tokens.
    f16x8 Sh[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        Sh[s][r] = (_Float16)S[2 * s][r];
        Sh[s][4 + r] = (_Float16)S[2 * s + 1][r];
      }
    const int tcol = wave * 16 + l16;   // column within the tile
    f32x4 Vn[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s <= (mt >> 1); ++s) {   // U = A v
        const f16x8 a = lds_f16x8(sA + (16 * mt + l16) * AS + 32 * s + 8 * gq);
        const f16x8 b = lds_f16x8(sVT + tcol * AS + 32 * s + 8 * gq);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {            // Vnew = U + (-W) S
        const uint16_t* row = sW + (16 * mt + l16) * QS + 32 * s + 4 * gq;
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(lds_f16_2x4(row, row + 16), Sh[s], acc, 0, 0, 0);
      }
      Vn[mt] = acc;
    }
    f16x8 Vh[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        Vh[s][r] = (_Float16)Vn[2 * s][r];
        Vh[s][4 + r] = (_Float16)Vn[2 * s + 1][r];
      }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {            // Qg S
        const uint16_t* row = sQ + (16 * mt + l16) * QS + 32 * s + 4 * gq;
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(lds_f16_2x4(row, row + 16), Sh[s], acc, 0, 0, 0);
      }
#pragma unroll
      for (int s = 0; s <= (mt >> 1); ++s) {   // + Aqk Vnew
        const uint16_t* row = sAqk + (16 * mt + l16) * AS + 32 * s + 4 * gq;
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(lds_f16_2x4(row, row + 16), Vh[s], acc, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * mt + 4 * gq + r;
        if (i < nvalid) p.o[((trow + i) * p.HV + hv) * KD + col] = uint16_t(bf16_rne(acc[r]));
      }
    }
#pragma unroll
    for (int rt = 0; rt < 8; ++rt) {           // S = e^{G_last} S + Kg^T Vnew
      f32x4 acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = S[rt][r] * sGam[16 * rt + 4 * gq + r];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint16_t* row = sKgT + (16 * rt + l16) * AS + 32 * s + 4 * gq;
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(lds_f16_2x4(row, row + 16), Vh[s], acc, 0, 0, 0);
      }
      S[rt] = acc;
    }
    __syncthreads();
  }

  float* sf = p.sfin + (int64_t(n) * p.HV + hv) * KD * KD;
#pragma unroll
  for (int rt = 0; rt < 8; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) sf[(16 * rt + 4 * gq + r) * KD + col] = S[rt][r];
}

template <int VT>
int launch(const Params& p, hipStream_t stream) {
  constexpr int NV = KD / VT;
  const int64_t units = int64_t(p.N) * p.HV;
  const int64_t blocks = (units + 7) / 8 * 8 * NV;
  if (blocks > 0x7fffffff) return KDA_ERR_SHAPE;
  static std::atomic<bool> configured{false};   // raise the dynamic LDS limit once
  if (!configured.load(std::memory_order_acquire)) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<VT>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, Lds<VT>::BYTES) != hipSuccess)
      return KDA_ERR_HIP;
    configured.store(true, std::memory_order_release);
  }
  hipLaunchKernelGGL(prefill_kernel<VT>, dim3(unsigned(blocks)), dim3(VT * 4), Lds<VT>::BYTES, stream, p);
  return launch_status();
}

}  // namespace

extern "C" int kda_chunk_prefill(const void* q, const void* k, const void* v, const float* g,
                                 const void* beta, const float* initial_state,
                                 const int32_t* cu_seqlens, int32_t num_seqs, int32_t B,
                                 int32_t T, int32_t H, int32_t HV, int32_t Kd, int32_t Vd,
                                 void* o, float* final_state, void* stream) {
  if (B < 1 || T < 0 || H < 1 || HV < 1 || HV % H != 0) return KDA_ERR_SHAPE;
  if (!final_state || (T > 0 && (!q || !k || !v || !g || !beta || !o))) return KDA_ERR_NULL;
  if (Kd != KD || Vd != KD) return KDA_ERR_UNSUPPORTED;
  if (cu_seqlens && (B != 1 || num_seqs < 1)) return KDA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(o) ||
      !aligned16(final_state) || (initial_state && !aligned16(initial_state)))
    return KDA_ERR_ALIGN;
  Params p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.g = g;
  p.beta = static_cast<const uint16_t*>(beta);
  p.s0 = initial_state;
  p.cu = cu_seqlens;
  p.o = static_cast<uint16_t*>(o);
  p.sfin = final_state;
  p.B = B;
  p.T = T;
  p.H = H;
  p.HV = HV;
  p.N = cu_seqlens ? num_seqs : B;
  // Fewer (sequence, head) units than compute units: split V in two tiles so
  // twice as many workgroups share the work.
  const int64_t units = int64_t(p.N) * HV;
  hipStream_t st = as_stream(stream);
  return units < 256 ? launch<64>(p, st) : launch<128>(p, st);
}
