// KDA chunked prefill (export kda_chunk_prefill).
//
// Page "KDA Chunk Prefill on Ascend A3": section "Function and tensor
// contract" (shapes, GQA head mapping) and section "Mathematical definition"
// (Q/K L2 normalisation; the chunk construction G, L, A = solve(I+L,
// diag(beta)), W, U, Qg, Kg, Aqk; the carry Vnew = U - W S, O = Qg S + Aqk
// Vnew, S = exp(G_last) S + Kg^T Vnew; chunk size 64 with a zero-padded last
// chunk).
//
// Design: one fused kernel, no workspace, one 512-thread workgroup (8 waves)
// per (sequence, value head).  Wave w owns state columns 16w..16w+15 and
// keeps that 128x16 slice of S in registers as float32 for the whole
// sequence (the state's columns evolve independently: column v of S only
// ever meets column v of the values).  For each 64-token chunk:
//   1. the raw q, k, g, beta and v of the chunk, prefetched into registers
//      while the previous chunk was computed, are normalised (bit-exact
//      routine shared with kda_qk_l2norm), scanned (G, kept in log2 units)
//      and staged in LDS; the loads for the next chunk are issued;
//   2. the gated L and Aqk, 16x16 blocks on MFMA;
//   3. T = (I+L)^-1 by blocked forward substitution in float32 (diagonal
//      blocks by substitution, off-diagonal blocks on fp32 MFMA), then
//      A = T diag(beta);
//   4. W = A (exp(G) k), Qg, Kg, exp(G_last);
//   5. each wave runs the carry for its columns on MFMA: U = A v and Vnew =
//      U - W S accumulate in float32 (U is never rounded), O = Qg S + Aqk
//      Vnew (staged in LDS, written with 16-byte stores), S = exp(G_last) S +
//      Kg^T Vnew.
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
constexpr int NW = 8;            // waves per workgroup
constexpr int NT = NW * 64;      // threads per workgroup
constexpr float LOG2E = 1.4426950408889634f;
constexpr float SCALE = 0.08838834764831845f;   // 128^-1/2
constexpr float SAFE_EXP2 = 120.0f;             // largest split-factor exponent (base 2)
constexpr float F16_EXP2 = 14.0f;               // largest split-factor exponent for fp16 operands

// LDS row strides (elements).  Row strides of 68 or 36 words put eight
// consecutive rows' 16-byte accesses in distinct bank groups.
constexpr int QS = 136;          // 16-bit [64][128] arrays
constexpr int GS = 132;          // fp32 [64][128] (G)
constexpr int OS = 136;          // bf16 [64][128] (o staging, in the G region)
constexpr int LS = 68;           // fp32 [64][64] arrays
constexpr int AS = 72;           // 16-bit [*][64] arrays

// LDS map (bytes).  Regions are reused across phases:
//   G    : fp32 G (phases 1-4), then bf16 o staging (phase 5)
//   U1   : fp32 L and T (phases 2-3), then fp16 -W and E^T (phases 4-5)
//   AREG : fp32 scan totals (phase 1), fp16 A (phases 3-5)
constexpr int OFF_Q = 0;                                  // bf16 q^, then fp16 Qg  [64][QS]
constexpr int OFF_K = OFF_Q + C * QS * 2;                 // bf16 k^                [64][QS]
constexpr int OFF_G = OFF_K + C * QS * 2;                 // fp32 G (log2 units)    [64][GS]
constexpr int OFF_U1 = OFF_G + C * GS * 4;
constexpr int OFF_L = OFF_U1;                             // fp32 L                 [64][LS]
constexpr int OFF_T = OFF_U1 + C * LS * 4;                // fp32 (I+L)^-1          [64][LS]
constexpr int OFF_W = OFF_U1;                             // fp16 -W                [64][QS]
constexpr int OFF_ET = OFF_U1 + C * QS * 2;               // fp16 (e^G k)^T         [128][AS]
constexpr int U1_BYTES = (2 * C * LS * 4 > C * QS * 2 + KD * AS * 2) ? 2 * C * LS * 4
                                                                     : C * QS * 2 + KD * AS * 2;
constexpr int OFF_AQK = OFF_U1 + U1_BYTES;                // fp16 Aqk               [64][AS]
constexpr int OFF_A = OFF_AQK + C * AS * 2;               // fp16 A [64][AS] / scan totals
constexpr int OFF_KGT = OFF_A + C * AS * 2;               // fp16 Kg^T              [128][AS]
constexpr int OFF_V = OFF_KGT + KD * AS * 2;              // fp16 v                 [64][QS]
constexpr int OFF_BETA = OFF_V + C * QS * 2;              // fp32 [64]
constexpr int OFF_GAM = OFF_BETA + C * 4;                 // fp32 [128]
constexpr int LDS_BYTES = OFF_GAM + KD * 4;
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
static_assert(C * AS * 2 >= 16 * KD * 4, "scan totals fit in the A region");
static_assert(C * GS * 4 >= C * OS * 2, "o staging fits in the G region");

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
  int T, H, HV, N;
};

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f16x8 lds_f16x8(const uint16_t* p) {
  return *reinterpret_cast<const f16x8*>(p);
}
// Storage position of contraction index c in the "permuted" LDS layout used
// for MFMA A operands whose B operand comes straight from a float32
// accumulator: within each group of 32, index 4g + e (e < 4) goes to 8g + e
// and index 16 + 4g + e goes to 8g + 4 + e, so the 8 values lane group g
// needs for one k-step are one contiguous 16-byte read.
__device__ __forceinline__ int perm32(int c) {
  const int cp = c & 31;
  return (c & ~31) + 8 * ((cp & 15) >> 2) + 4 * (cp >> 4) + (cp & 3);
}

// Value of `v` in lane `src` (0..3) of each lane's quad.
__device__ __forceinline__ float quad_bcast(float v, int src) {
  const int x = __builtin_bit_cast(int, v);
  int r;
  switch (src) {
    case 0: r = __builtin_amdgcn_update_dpp(0, x, 0x00, 0xf, 0xf, false); break;
    case 1: r = __builtin_amdgcn_update_dpp(0, x, 0x55, 0xf, 0xf, false); break;
    case 2: r = __builtin_amdgcn_update_dpp(0, x, 0xAA, 0xf, 0xf, false); break;
    default: r = __builtin_amdgcn_update_dpp(0, x, 0xFF, 0xf, 0xf, false); break;
  }
  return __builtin_bit_cast(float, r);
}
__device__ __forceinline__ uint16_t f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  return uint32_t(f16_bits(lo)) | (uint32_t(f16_bits(hi)) << 16);
}
__device__ __forceinline__ void unpack_bf16x8(const uint4& x, float* f) {
  f[0] = bf16lo(x.x); f[1] = bf16hi(x.x);
  f[2] = bf16lo(x.y); f[3] = bf16hi(x.y);
  f[4] = bf16lo(x.z); f[5] = bf16hi(x.z);
  f[6] = bf16lo(x.w); f[7] = bf16hi(x.w);
}

// Raw inputs of one chunk held in registers (prefetch buffer).
//   qk[m]: row rg + 32m of the 128 stacked rows (q rows 0..63, k rows 64..127),
//          8 bf16 at column 8*l16, with rg = tid/16, l16 = tid%16
//   gv[r]: g of token 4*seg + r, channels 4*c4..4*c4+3 (seg = tid/32, c4 = tid%32)
//   vv[m]: v of token tid/16 + 32m, columns 8*(tid%16)..+7
struct Raw {
  uint4 qk[4];
  float4 gv[4];
  uint4 vv[2];
  float beta;
};

__device__ __forceinline__ void load_raw(Raw& R, const Params& p, int64_t trow, int nvalid, int hq,
                                         int hv, int tid) {
  const int rg = tid >> 4, l16 = tid & 15;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int i = (rg + 32 * m) & (C - 1);
    const uint16_t* base = (m < 2) ? p.q : p.k;
    R.qk[m] = make_uint4(0u, 0u, 0u, 0u);
    if (i < nvalid) R.qk[m] = *reinterpret_cast<const uint4*>(base + ((trow + i) * p.H + hq) * KD + 8 * l16);
  }
  const int seg = tid >> 5, c4 = tid & 31;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 4 * seg + r;
    R.gv[r] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < nvalid) R.gv[r] = *reinterpret_cast<const float4*>(p.g + ((trow + i) * p.HV + hv) * KD + 4 * c4);
  }
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int i = rg + 32 * m;
    R.vv[m] = make_uint4(0u, 0u, 0u, 0u);
    if (i < nvalid) R.vv[m] = *reinterpret_cast<const uint4*>(p.v + ((trow + i) * p.HV + hv) * KD + 8 * l16);
  }
  R.beta = 0.f;
  if (tid < nvalid) R.beta = bf16f(p.beta[(trow + tid) * p.HV + hv]);
}

__global__ __launch_bounds__(NT) void prefill_kernel(Params p) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* sQ = reinterpret_cast<uint16_t*>(smem + OFF_Q);
  uint16_t* sK = reinterpret_cast<uint16_t*>(smem + OFF_K);
  float* sG = reinterpret_cast<float*>(smem + OFF_G);
  uint16_t* sO = reinterpret_cast<uint16_t*>(smem + OFF_G);
  float* sL = reinterpret_cast<float*>(smem + OFF_L);
  float* sT = reinterpret_cast<float*>(smem + OFF_T);
  uint16_t* sW = reinterpret_cast<uint16_t*>(smem + OFF_W);
  uint16_t* sET = reinterpret_cast<uint16_t*>(smem + OFF_ET);
  uint16_t* sAqk = reinterpret_cast<uint16_t*>(smem + OFF_AQK);
  uint16_t* sA = reinterpret_cast<uint16_t*>(smem + OFF_A);
  float* sScr = reinterpret_cast<float*>(smem + OFF_A);
  uint16_t* sKgT = reinterpret_cast<uint16_t*>(smem + OFF_KGT);
  uint16_t* sV = reinterpret_cast<uint16_t*>(smem + OFF_V);
  float* sBeta = reinterpret_cast<float*>(smem + OFF_BETA);
  float* sGam = reinterpret_cast<float*>(smem + OFF_GAM);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int gq = lane >> 4;

  const int unit = blockIdx.x;
  if (unit >= p.N * p.HV) return;
  const int n = unit / p.HV;
  const int hv = unit % p.HV;
  const int hq = hv / (p.HV / p.H);

  int64_t tok0;   // row of the sequence's first token in the [B*T] token axis
  int len;
  if (p.cu) {
    tok0 = p.cu[n];
    len = p.cu[n + 1] - p.cu[n];
  } else {
    tok0 = int64_t(n) * p.T;
    len = p.T;
  }

  const int col = wave * 16 + l16;               // this lane's state column
  f32x4 S[8];                                    // rows 16rt + 4gq + r of column `col`
  {
    const float* s0 = p.s0 ? p.s0 + (int64_t(n) * p.HV + hv) * KD * KD : nullptr;
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) S[rt][r] = s0 ? s0[(16 * rt + 4 * gq + r) * KD + col] : 0.f;
  }

  Raw R;
  if (len > 0) load_raw(R, p, tok0, min(C, len), hq, hv, tid);

  for (int c0 = 0; c0 < len; c0 += C) {
    const int nvalid = min(C, len - c0);
    const int64_t trow = tok0 + c0;              // token row of chunk position 0

    // ---------------------------------------------------------- phase 1
    {
      const int rg = tid >> 4;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint4 y = l2norm_row16(R.qk[m]);
        *reinterpret_cast<uint4*>(((m < 2) ? sQ : sK) + ((rg + 32 * m) & (C - 1)) * QS + 8 * l16) = y;
        __builtin_amdgcn_sched_barrier(0);   // one row at a time keeps register use low
      }
      // v (bf16 -> fp16), row-major.
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        float f[8];
        unpack_bf16x8(R.vv[m], f);
        *reinterpret_cast<uint4*>(sV + (rg + 32 * m) * QS + 8 * l16) =
            make_uint4(pack_f16(f[0], f[1]), pack_f16(f[2], f[3]), pack_f16(f[4], f[5]), pack_f16(f[6], f[7]));
      }
      if (tid < C) sBeta[tid] = R.beta;
      // g in log2 units, inclusive scan over the 4 tokens this thread holds,
      // then across the 16 four-token segments through LDS.
      const int seg = tid >> 5, c4 = tid & 31;
      float4 gs[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        gs[r].x = R.gv[r].x * LOG2E + (r ? gs[r - 1].x : 0.f);
        gs[r].y = R.gv[r].y * LOG2E + (r ? gs[r - 1].y : 0.f);
        gs[r].z = R.gv[r].z * LOG2E + (r ? gs[r - 1].z : 0.f);
        gs[r].w = R.gv[r].w * LOG2E + (r ? gs[r - 1].w : 0.f);
      }
      *reinterpret_cast<float4*>(sScr + seg * KD + 4 * c4) = gs[3];
      __syncthreads();
      // The raw registers are consumed: prefetch the next chunk.
      if (c0 + C < len) load_raw(R, p, trow + C, min(C, len - c0 - C), hq, hv, tid);
      float4 off = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int s2 = 0; s2 < seg; ++s2) {
        const float4 t = *reinterpret_cast<const float4*>(sScr + s2 * KD + 4 * c4);
        off.x += t.x;
        off.y += t.y;
        off.z += t.z;
        off.w += t.w;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *reinterpret_cast<float4*>(sG + (4 * seg + r) * GS + 4 * c4) =
            make_float4(gs[r].x + off.x, gs[r].y + off.y, gs[r].z + off.z, gs[r].w + off.w);
    }
    __syncthreads();

    // ---------------------------------------------------------- phase 2: L, Aqk
    // The 10 blocks on or below the diagonal over 8 waves; waves 2..7 also
    // zero one strictly-upper block of Aqk each.
    {
      if (wave >= 2) {
        const int ub = wave - 2;
        const int UI = ub < 3 ? 0 : (ub < 5 ? 1 : 2);
        const int UJ = ub < 3 ? ub + 1 : (ub < 5 ? ub - 1 : 3);
#pragma unroll
        for (int r = 0; r < 4; ++r) sAqk[(16 * UI + 4 * gq + r) * AS + perm32(16 * UJ + l16)] = 0;
      }
      for (int pb = wave; pb < 10; pb += NW) {
        // blocks ordered (3,0) (3,1) (3,2) (3,3) (2,0) (2,1) (2,2) (1,0) (1,1) (0,0)
        const int I = pb < 4 ? 3 : (pb < 7 ? 2 : (pb < 9 ? 1 : 0));
        const int J = pb < 4 ? pb : (pb < 7 ? pb - 4 : (pb < 9 ? pb - 7 : 0));
        const int ref = (J < I) ? 16 * I : 16 * I + 8;
        const int i = 16 * I + l16;     // operand row (A side)
        const int j = 16 * J + l16;     // operand row (B side)
        // Largest split-factor exponent of this lane's entries (<= 0 below the
        // diagonal, so only diagonal blocks need the check).
        float emax = 0.f;
        if (J == I) {
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const int ch0 = 32 * s + 8 * gq;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const float4 gi = *reinterpret_cast<const float4*>(sG + i * GS + ch0 + 4 * h);
              const float4 gj = *reinterpret_cast<const float4*>(sG + j * GS + ch0 + 4 * h);
              const float4 gr = *reinterpret_cast<const float4*>(sG + ref * GS + ch0 + 4 * h);
              emax = fmaxf(emax, fmaxf(fmaxf(gi.x - gr.x, gi.y - gr.y), fmaxf(gi.z - gr.z, gi.w - gr.w)));
              emax = fmaxf(emax, fmaxf(fmaxf(gr.x - gj.x, gr.y - gj.y), fmaxf(gr.z - gj.z, gr.w - gj.w)));
            }
          }
        }
        f32x4 accL = {0.f, 0.f, 0.f, 0.f};
        f32x4 accQ = {0.f, 0.f, 0.f, 0.f};
        const bool wide = __any(emax > F16_EXP2);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int ch0 = 32 * s + 8 * gq;
          float ki[8], qi[8], kj[8];
          unpack_bf16x8(*reinterpret_cast<const uint4*>(sK + i * QS + ch0), ki);
          unpack_bf16x8(*reinterpret_cast<const uint4*>(sQ + i * QS + ch0), qi);
          unpack_bf16x8(*reinterpret_cast<const uint4*>(sK + j * QS + ch0), kj);
          float kr[8], qr[8], kc[8];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float4 gi4 = *reinterpret_cast<const float4*>(sG + i * GS + ch0 + 4 * h);
            const float4 gj4 = *reinterpret_cast<const float4*>(sG + j * GS + ch0 + 4 * h);
            const float4 gr4 = *reinterpret_cast<const float4*>(sG + ref * GS + ch0 + 4 * h);
            const float gi[4] = {gi4.x, gi4.y, gi4.z, gi4.w};
            const float gj[4] = {gj4.x, gj4.y, gj4.z, gj4.w};
            const float gr[4] = {gr4.x, gr4.y, gr4.z, gr4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float fr = ex2(gi[e] - gr[e]);
              const float fc = ex2(gr[e] - gj[e]);
              kr[4 * h + e] = ki[4 * h + e] * fr;
              qr[4 * h + e] = qi[4 * h + e] * fr;
              kc[4 * h + e] = kj[4 * h + e] * fc;
            }
          }
          if (!wide) {
            f16x8 a, b, c;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              a[e] = (_Float16)kr[e];
              b[e] = (_Float16)qr[e];
              c[e] = (_Float16)kc[e];
            }
            accL = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, c, accL, 0, 0, 0);
            accQ = __builtin_amdgcn_mfma_f32_16x16x32_f16(b, c, accQ, 0, 0, 0);
          } else {
            // Steep decay inside a diagonal block: bf16 operands keep the range.
            bf16x8 a, b, c;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              a[e] = (__bf16)kr[e];
              b[e] = (__bf16)qr[e];
              c[e] = (__bf16)kc[e];
            }
            accL = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, c, accL, 0, 0, 0);
            accQ = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, c, accQ, 0, 0, 0);
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
                const float kjf = bf16f(sK[jc * QS + ch]) * f;
                aL = fmaf(bf16f(sK[ir * QS + ch]), kjf, aL);
                aQ = fmaf(bf16f(sQ[ir * QS + ch]), kjf, aQ);
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
          sAqk[ir * AS + perm32(jc)] = f16_bits((jc <= ir) ? SCALE * accQ[r] : 0.f);
        }
      }
    }
    __syncthreads();

    // ---------------------------------------------------------- phase 3: solve
    // T = (I + L)^-1, unit lower triangular.
    // Diagonal 16x16 blocks: wave b < 4 inverts block b.  Lane 4*cc + h holds
    // rows 4h..4h+3 of column cc and the matching rows of L in registers;
    // column-oriented forward substitution broadcasts x[m] within the quad.
    if (wave < 4) {
      const int blk = wave;
      const int cc = lane >> 2;
      const int h = lane & 3;
      float Lr[4][16];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ii = 4 * h + r;
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4) {
          const float4 l4 = *reinterpret_cast<const float4*>(sL + (16 * blk + ii) * LS + 16 * blk + 4 * m4);
          Lr[r][4 * m4 + 0] = (4 * m4 + 0 < ii) ? l4.x : 0.f;
          Lr[r][4 * m4 + 1] = (4 * m4 + 1 < ii) ? l4.y : 0.f;
          Lr[r][4 * m4 + 2] = (4 * m4 + 2 < ii) ? l4.z : 0.f;
          Lr[r][4 * m4 + 3] = (4 * m4 + 3 < ii) ? l4.w : 0.f;
        }
      }
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = (4 * h + r == cc) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < 15; ++m) {
        // x[m] lives in quad lane m/4, register m%4; broadcast it to the quad.
        const float xm = quad_bcast(x[m & 3], m >> 2);
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = fmaf(-Lr[r][m], xm, x[r]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) sT[(16 * blk + 4 * h + r) * LS + 16 * blk + cc] = x[r];
    }
    __syncthreads();
    // Off-diagonal blocks, one block row at a time, on fp32 MFMA (16x16x4):
    //   P_IJ = sum_{M=J}^{I-1} L_IM T_MJ,   T_IJ = -T_II P_IJ.
    // For the second product the contraction index of k-step s in lane group
    // gq is 4gq + s, which is where P's accumulator already holds it.
    for (int I = 1; I < 4; ++I) {
      if (wave < I) {
        const int J = wave;
        f32x4 P = {0.f, 0.f, 0.f, 0.f};
        for (int M = J; M < I; ++M) {
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const float a = sL[(16 * I + l16) * LS + 16 * M + 4 * s + gq];
            const float b = sT[(16 * M + 4 * s + gq) * LS + 16 * J + l16];
            P = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, P, 0, 0, 0);
          }
        }
        f32x4 X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const float a = -sT[(16 * I + l16) * LS + 16 * I + 4 * gq + s];
          X = __builtin_amdgcn_mfma_f32_16x16x4f32(a, P[s], X, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) sT[(16 * I + 4 * gq + r) * LS + 16 * J + l16] = X[r];
      }
      __syncthreads();
    }
    // A = T diag(beta), lower triangular, as fp16 (8 entries per thread).
    {
      const int ii = tid >> 3;
      const int j0 = 8 * (tid & 7);
      const float4 t0 = *reinterpret_cast<const float4*>(sT + ii * LS + j0);
      const float4 t1 = *reinterpret_cast<const float4*>(sT + ii * LS + j0 + 4);
      const float4 b0 = *reinterpret_cast<const float4*>(sBeta + j0);
      const float4 b1 = *reinterpret_cast<const float4*>(sBeta + j0 + 4);
      const float tv[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
      const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
      float a[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] = (j0 + e <= ii) ? tv[e] * bv[e] : 0.f;
      *reinterpret_cast<uint4*>(sA + ii * AS + j0) =
          make_uint4(pack_f16(a[0], a[1]), pack_f16(a[2], a[3]), pack_f16(a[4], a[5]), pack_f16(a[6], a[7]));
    }
    if (tid < KD) sGam[tid] = ex2(sG[(C - 1) * GS + tid]);
    __syncthreads();

    // ---------------------------------------------------------- phase 4: E, Kg, Qg, W
    // Thread t handles channels c2, c2+1 (c2 = 2*(t%64)) for tokens
    // 8*(t/64)..+7.
    uint32_t qg_pk[8];   // Qg of this thread's entries, stored after the barrier
    {
      const int c2 = 2 * (tid & 63);
      const int j0 = 8 * (tid >> 6);
      const float2 glast = *reinterpret_cast<const float2*>(sG + (C - 1) * GS + c2);
      float ev0[8], ev1[8], kv0[8], kv1[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int jj = j0 + e;
        const float2 gj = *reinterpret_cast<const float2*>(sG + jj * GS + c2);
        const uint32_t kk = *reinterpret_cast<const uint32_t*>(sK + jj * QS + c2);
        const uint32_t qq = *reinterpret_cast<const uint32_t*>(sQ + jj * QS + c2);
        const float eg0 = ex2(gj.x), eg1 = ex2(gj.y);
        const float k0 = bf16lo(kk), k1 = bf16hi(kk);
        ev0[e] = k0 * eg0;
        ev1[e] = k1 * eg1;
        kv0[e] = k0 * ex2(glast.x - gj.x);
        kv1[e] = k1 * ex2(glast.y - gj.y);
        qg_pk[e] = pack_f16(SCALE * bf16lo(qq) * eg0, SCALE * bf16hi(qq) * eg1);
      }
      *reinterpret_cast<uint4*>(sET + c2 * AS + j0) =
          make_uint4(pack_f16(ev0[0], ev0[1]), pack_f16(ev0[2], ev0[3]), pack_f16(ev0[4], ev0[5]), pack_f16(ev0[6], ev0[7]));
      *reinterpret_cast<uint4*>(sET + (c2 + 1) * AS + j0) =
          make_uint4(pack_f16(ev1[0], ev1[1]), pack_f16(ev1[2], ev1[3]), pack_f16(ev1[4], ev1[5]), pack_f16(ev1[6], ev1[7]));
      // Kg^T in the permuted token layout: tokens j0..j0+3 and j0+4..j0+7 each
      // land as one contiguous 8-byte group.
      const int pj0 = perm32(j0), pj4 = perm32(j0 + 4);
      *reinterpret_cast<uint2*>(sKgT + c2 * AS + pj0) = make_uint2(pack_f16(kv0[0], kv0[1]), pack_f16(kv0[2], kv0[3]));
      *reinterpret_cast<uint2*>(sKgT + c2 * AS + pj4) = make_uint2(pack_f16(kv0[4], kv0[5]), pack_f16(kv0[6], kv0[7]));
      *reinterpret_cast<uint2*>(sKgT + (c2 + 1) * AS + pj0) = make_uint2(pack_f16(kv1[0], kv1[1]), pack_f16(kv1[2], kv1[3]));
      *reinterpret_cast<uint2*>(sKgT + (c2 + 1) * AS + pj4) = make_uint2(pack_f16(kv1[4], kv1[5]), pack_f16(kv1[6], kv1[7]));
    }
    __syncthreads();
    // Qg (over q^, now no longer read) in the permuted channel layout; c2 and
    // c2 + 1 stay adjacent there.
    {
      const int pc = perm32(2 * (tid & 63));
      const int j0 = 8 * (tid >> 6);
#pragma unroll
      for (int e = 0; e < 8; ++e) *reinterpret_cast<uint32_t*>(sQ + (j0 + e) * QS + pc) = qg_pk[e];
    }
    // W = A (e^G k): 4 x 8 output tiles, 4 per wave; A is lower triangular.
    // -W is stored in the permuted channel layout.
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int pt = wave + NW * q4;
      const int mt = pt >> 3;
      const int nt = pt & 7;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int s = 0; s <= (mt >> 1); ++s) {
        const f16x8 a = lds_f16x8(sA + (16 * mt + l16) * AS + 32 * s + 8 * gq);
        const f16x8 b = lds_f16x8(sET + (16 * nt + l16) * AS + 32 * s + 8 * gq);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
      }
      const int pc = perm32(16 * nt + l16);
#pragma unroll
      for (int r = 0; r < 4; ++r) sW[(16 * mt + 4 * gq + r) * QS + pc] = f16_bits(-acc[r]);
    }
    __syncthreads();

    // ---------------------------------------------------------- phase 5: carry
    // Contraction orders: for products with S the channel index of k-slot
    // (gq, e) is 32s + 4gq + e (e < 4) or 32s + 16 + 4gq + (e - 4), which is
    // exactly where the float32 S accumulator already holds it; products with
    // Vnew use the same permutation over tokens.
    {
      f16x8 Sh[4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          Sh[s][r] = (_Float16)S[2 * s][r];
          Sh[s][4 + r] = (_Float16)S[2 * s + 1][r];
        }
      // v as the B operand of U = A v: tokens 32s + 8gq + e of column `col`.
      f16x8 Vv[2];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          Vv[s][e] = __builtin_bit_cast(_Float16, sV[(32 * s + 8 * gq + e) * QS + col]);
      // U = A v, then Vnew = U + (-W) S; the four token tiles are independent
      // accumulation chains, interleaved.
      f32x4 Vn[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) Vn[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          if (s <= (mt >> 1))
            Vn[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                lds_f16x8(sA + (16 * mt + l16) * AS + 32 * s + 8 * gq), Vv[s], Vn[mt], 0, 0, 0);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          Vn[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              lds_f16x8(sW + (16 * mt + l16) * QS + 32 * s + 8 * gq), Sh[s], Vn[mt], 0, 0, 0);
      f16x8 Vh[2];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          Vh[s][r] = (_Float16)Vn[2 * s][r];
          Vh[s][4 + r] = (_Float16)Vn[2 * s + 1][r];
        }
      // O = Qg S + Aqk Vnew.
      f32x4 Ot[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) Ot[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          Ot[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              lds_f16x8(sQ + (16 * mt + l16) * QS + 32 * s + 8 * gq), Sh[s], Ot[mt], 0, 0, 0);
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          if (s <= (mt >> 1))
            Ot[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                lds_f16x8(sAqk + (16 * mt + l16) * AS + 32 * s + 8 * gq), Vh[s], Ot[mt], 0, 0, 0);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) sO[(16 * mt + 4 * gq + r) * OS + col] = uint16_t(bf16_rne(Ot[mt][r]));
      // S = e^{G_last} S + Kg^T Vnew; eight independent row tiles.
#pragma unroll
      for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[rt][r] *= sGam[16 * rt + 4 * gq + r];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
          S[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              lds_f16x8(sKgT + (16 * rt + l16) * AS + 32 * s + 8 * gq), Vh[s], S[rt], 0, 0, 0);
    }
    __syncthreads();
    // o: 16-byte stores of the staged bf16 tile (two per thread).
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int i = (tid >> 4) + 32 * m;
      if (i < nvalid)
        *reinterpret_cast<uint4*>(p.o + ((trow + i) * p.HV + hv) * KD + 8 * l16) =
            *reinterpret_cast<const uint4*>(sO + i * OS + 8 * l16);
    }
  }

  float* sf = p.sfin + (int64_t(n) * p.HV + hv) * KD * KD;
#pragma unroll
  for (int rt = 0; rt < 8; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) sf[(16 * rt + 4 * gq + r) * KD + col] = S[rt][r];
}

int launch(const Params& p, hipStream_t stream) {
  const int64_t blocks = int64_t(p.N) * p.HV;
  if (blocks > 0x7fffffff) return KDA_ERR_SHAPE;
  static std::atomic<bool> configured{false};   // raise the dynamic LDS limit once
  if (!configured.load(std::memory_order_acquire)) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES) != hipSuccess)
      return KDA_ERR_HIP;
    configured.store(true, std::memory_order_release);
  }
  hipLaunchKernelGGL(prefill_kernel, dim3(unsigned(blocks)), dim3(NT), LDS_BYTES, stream, p);
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
  p.T = T;
  p.H = H;
  p.HV = HV;
  p.N = cu_seqlens ? num_seqs : B;
  return launch(p, as_stream(stream));
}
