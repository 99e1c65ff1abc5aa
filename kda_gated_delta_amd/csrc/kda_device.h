// Device helpers shared by the KDA kernels (gfx950 / CDNA4, wave64).
//
// The bit-exact row L2 normalisation lives here so that the standalone
// export, the prefill kernel and the decode kernel produce identical bf16
// values.  Definition (page "KDA Chunk Prefill on Ascend A3", section
// "Mathematical definition"): y = bf16(x / sqrt(sum(x*x) + 1e-6)) in float32,
// with the sum read as the exact sum of the float32 squares rounded once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kHead = 128;        // K == V
constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16 bits

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16f(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// float32 -> bfloat16 bits, round to nearest, ties to even (exact for
// subnormals and infinities; NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

// ---------------------------------------------------------------- exact sums

// Error-free sum: a + b = s + e exactly.
__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
  s = a + b;
  double bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}

// Neighbouring float32 of a finite r, upwards or downwards.
__device__ __forceinline__ float next_f32(float r, bool up) {
  if (r == 0.0f) return up ? __uint_as_float(1u) : -__uint_as_float(1u);
  uint32_t u = __float_as_uint(r);
  const bool grow = (r > 0.0f) == up;   // moving away from zero
  return __uint_as_float(grow ? u + 1u : u - 1u);
}

// Correct float32 rounding (nearest-even) of hi + lo, where the pair holds
// the exact value.  After renormalisation |lo| <= ulp64(hi)/2, so only an
// exactly-midway hi can be decided by lo.
__device__ __forceinline__ float dd_to_f32(double hi, double lo) {
  double s = hi + lo;
  double c = lo - (s - hi);
  float r = (float)s;
  if ((double)r == s || s == 0.0) return r;
  float n = next_f32(r, s > (double)r);
  double mid = 0.5 * ((double)r + (double)n);
  if (s == mid && c != 0.0) {
    bool toward_n = (c > 0.0) == ((double)n > (double)r);
    if (toward_n) return n;
  }
  return r;
}

// ---------------------------------------------------------------- row norm

// Normalise one row of 128 bf16 held by a 16-lane group (lanes sharing
// lane/16): each lane holds 8 consecutive elements packed in `x`.  Every
// lane of the wave must call this (cross-lane shuffles).  Returns the 8
// normalised bf16 values, packed the same way.
//
// Sum of squares: each square of a bf16 value is exact in float32.  When the
// row's nonzero magnitudes span at most 2^15 (biased exponents differ by
// <= 15), every partial sum of the squares is exact in float64, so the
// float64 tree sum is exact in any order and one conversion rounds it
// correctly.  Otherwise (rare) the whole wave takes an error-free
// double-double path, exact while the span is at most 2^38.
//
// Division: with d the correctly rounded float32 square root, the float64
// product x * RN64(1/d) lies within 2^-51.9 relative of x/d, while x/d (x
// has 8 significant bits) is at least 2^-49 relative away from every
// float32 rounding midpoint; converting the product to float32 therefore
// gives the correctly rounded float32 quotient.  The square root is taken
// in float64 and rounded to float32, which is correctly rounded because
// 53 >= 2*24 + 2.
__device__ __forceinline__ uint4 l2norm_row16(uint4 x) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  float xf[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xf[2 * i] = bf16lo(w[i]);
    xf[2 * i + 1] = bf16hi(w[i]);
  }
  double s = 0.0;
  int emax = 0, emin = 255;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float sq = xf[i] * xf[i];
    s += (double)sq;
    uint32_t mag = (__float_as_uint(xf[i]) >> 16) & 0x7fffu;
    int e = int(mag >> 7);
    e = e < 1 ? 1 : e;
    if (mag != 0u) {
      emax = emax > e ? emax : e;
      emin = emin < e ? emin : e;
    }
  }
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) {
    s += __shfl_xor(s, off, 64);
    int a = __shfl_xor(emax, off, 64);
    int b = __shfl_xor(emin, off, 64);
    emax = emax > a ? emax : a;
    emin = emin < b ? emin : b;
  }
  const bool exact = (emax == 0) || (emax - emin <= 15);
  float s32 = (float)s;
  if (!__all(exact)) {
    double hi = 0.0, lo = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      double t, e;
      two_sum(hi, (double)(xf[i] * xf[i]), t, e);
      hi = t;
      lo += e;
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      double oh = __shfl_xor(hi, off, 64);
      double ol = __shfl_xor(lo, off, 64);
      double t, e;
      two_sum(hi, oh, t, e);
      double l = lo + ol + e;
      hi = t + l;
      lo = l - (hi - t);
    }
    if (!exact) s32 = dd_to_f32(hi, lo);
  }
  const float t = s32 + 1e-6f;
  const float d = (float)__builtin_sqrt((double)t);
  const double r = 1.0 / (double)d;
  uint4 y;
  y.x = pack_bf16((float)((double)xf[0] * r), (float)((double)xf[1] * r));
  y.y = pack_bf16((float)((double)xf[2] * r), (float)((double)xf[3] * r));
  y.z = pack_bf16((float)((double)xf[4] * r), (float)((double)xf[5] * r));
  y.w = pack_bf16((float)((double)xf[6] * r), (float)((double)xf[7] * r));
  return y;
}

}  // namespace kda
