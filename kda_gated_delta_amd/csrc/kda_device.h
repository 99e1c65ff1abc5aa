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

// ---------------------------------------------------------------- barriers

// Workgroup barrier for LDS traffic only.  __syncthreads() also fences
// global memory, which makes every wave wait for all of its outstanding
// global loads and stores -- including prefetches meant to stay in flight
// across the barrier.  Here the compiler is kept from moving memory accesses
// across the barrier, the wave waits for its own LDS operations, and the
// hardware barrier does the rest.  Global data shared through LDS by direct
// loads must be waited for (vmcnt) by the caller before this.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---------------------------------------------------------------- bf16 bits

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16f(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// float32 pair -> packed bf16 (lo in bits 0..15), round to nearest, ties
// to even: the hardware conversion v_cvt_pk_bf16_f32, checked on MI355X
// against an integer round-to-nearest-even over all 2^32 float32 inputs
// (identical, subnormals and infinities included; NaN stays NaN).
//
// pack_bf16 is the compiler-visible form, for any float32 input -- in
// particular MFMA results, whose readers need wait states that the compiler
// inserts only for instructions it can see.  cvt_pk_bf16 is the same
// instruction in inline assembly, used only where the inputs come from a
// float64 -> float32 rounding by ordinary vector instructions: there it
// keeps the compiler from merging the two roundings into one.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  uint32_t r;
  asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(r) : "v"(lo), "v"(hi));
  return r;
}

// ---------------------------------------------------------------- streaming access

// 16-byte global store with the nontemporal hint, for data that is written
// once and read back only after it has long left the caches.
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_nt(uint4* p, const uint4& v) {
  const u32x4_nt w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4_nt*>(p));
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

// ---------------------------------------------------------------- row reductions

// All-reduce across the 16 lanes of a DPP row (lanes sharing lane/16), with
// register-only DPP moves: swap neighbours, swap pairs, then rotate the row
// by 4 and by 8.  Every lane ends with the reduction of its row.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t x) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(x), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp64(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = dpp32<CTRL>(uint32_t(u));
  const uint32_t hi = dpp32<CTRL>(uint32_t(u >> 32));
  return __builtin_bit_cast(double, (uint64_t(hi) << 32) | lo);
}
constexpr int kDppXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppRor4 = 0x124;   // row_ror:4
constexpr int kDppRor8 = 0x128;   // row_ror:8

__device__ __forceinline__ double row16_sum(double x) {
  x += dpp64<kDppXor1>(x);
  x += dpp64<kDppXor2>(x);
  x += dpp64<kDppRor4>(x);
  x += dpp64<kDppRor8>(x);
  return x;
}
__device__ __forceinline__ int row16_max(int x) {
  x = max(x, int(dpp32<kDppXor1>(uint32_t(x))));
  x = max(x, int(dpp32<kDppXor2>(uint32_t(x))));
  x = max(x, int(dpp32<kDppRor4>(uint32_t(x))));
  x = max(x, int(dpp32<kDppRor8>(uint32_t(x))));
  return x;
}
__device__ __forceinline__ int row16_min(int x) {
  x = min(x, int(dpp32<kDppXor1>(uint32_t(x))));
  x = min(x, int(dpp32<kDppXor2>(uint32_t(x))));
  x = min(x, int(dpp32<kDppRor4>(uint32_t(x))));
  x = min(x, int(dpp32<kDppRor8>(uint32_t(x))));
  return x;
}

constexpr int kDppHalfMirror = 0x141;   // row_half_mirror: lane i <-> 7 - i within 8 lanes

// All-reduce across 8-lane groups (lanes sharing lane/8): neighbours, pairs,
// then the mirrored quad.
__device__ __forceinline__ double row8_sum(double x) {
  x += dpp64<kDppXor1>(x);
  x += dpp64<kDppXor2>(x);
  x += dpp64<kDppHalfMirror>(x);
  return x;
}
__device__ __forceinline__ int row8_max(int x) {
  x = max(x, int(dpp32<kDppXor1>(uint32_t(x))));
  x = max(x, int(dpp32<kDppXor2>(uint32_t(x))));
  x = max(x, int(dpp32<kDppHalfMirror>(uint32_t(x))));
  return x;
}
__device__ __forceinline__ int row8_min(int x) {
  x = min(x, int(dpp32<kDppXor1>(uint32_t(x))));
  x = min(x, int(dpp32<kDppXor2>(uint32_t(x))));
  x = min(x, int(dpp32<kDppHalfMirror>(uint32_t(x))));
  return x;
}

// ---------------------------------------------------------------- row norm

// Normalise one row of 128 bf16 held by a 16-lane group (lanes sharing
// lane/16): each lane holds 8 consecutive elements packed in `x`.  Every
// lane of the wave must call this (cross-lane operations).  Returns the 8
// normalised bf16 values, packed the same way.
//
// Sum of squares: each square of a bf16 value is exact in float32.  When the
// row's nonzero magnitudes span at most 2^15 (biased exponents differ by
// <= 15), every partial sum of the squares is exact in float64, so the
// float64 sum is exact in any order (each lane of the row may add in its own
// order and all get the same value) and one conversion rounds it correctly.
// Otherwise (rare) the whole wave takes an error-free double-double path,
// exact while the span is at most 2^38; its result is taken from the row's
// first lane so that every lane of the row divides by the same value.
//
// Division: with d the correctly rounded float32 square root, the float64
// product x * RN64(1/d) lies within 2^-51.9 relative of x/d, while x/d (x
// has 8 significant bits) is at least 2^-49 relative away from every
// float32 rounding midpoint; converting the product to float32 therefore
// gives the correctly rounded float32 quotient.  The square root is taken
// in float64 and rounded to float32, which is correctly rounded because
// 53 >= 2*24 + 2.
__device__ __forceinline__ uint4 l2norm_row16(uint4 x) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  double xd[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xd[2 * i] = (double)bf16lo(w[i]);
    xd[2 * i + 1] = (double)bf16hi(w[i]);
  }
  // Largest magnitude and smallest nonzero magnitude (bf16 bit patterns
  // order like their values), two elements per packed 16-bit operation.
  u16x2 mx = {0, 0};
  u16x2 mn = {0xffff, 0xffff};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u16x2 m = __builtin_bit_cast(u16x2, w[i] & 0x7fff7fffu);
    mx = __builtin_elementwise_max(mx, m);
    mn = __builtin_elementwise_min(mn, m - (u16x2){1, 1});   // zero wraps to 0xffff
  }
  int emax = int(mx[0] > mx[1] ? mx[0] : mx[1]);           // magnitude bits
  int emin = int(mn[0] < mn[1] ? mn[0] : mn[1]) + 1;       // 0x10000 if all zero
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) s = fma(xd[i], xd[i], s);    // x*x is exact in float32 and float64
  s = row16_sum(s);
  emax = row16_max(emax) >> 7;                              // biased exponents
  emin = row16_min(emin) >> 7;
  const bool exact = (emax == 0 && emin == 512) || (max(emax, 1) - max(emin, 1) <= 15);
  float s32 = (float)s;
  if (!__all(exact)) {
    double hi = 0.0, lo = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      double t, e;
      two_sum(hi, xd[i] * xd[i], t, e);
      hi = t;
      lo += e;
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const double oh = __shfl_xor(hi, off, 64);
      const double ol = __shfl_xor(lo, off, 64);
      double t, e;
      two_sum(hi, oh, t, e);
      const double l = lo + ol + e;
      hi = t + l;
      lo = l - (hi - t);
    }
    const float r = __shfl(dd_to_f32(hi, lo), (threadIdx.x & 63) & ~15, 64);
    if (!exact) s32 = r;
  }
  const float t = s32 + 1e-6f;
  const float d = (float)__builtin_sqrt((double)t);
  const double r = 1.0 / (double)d;
  // Round the float32 quotient to bf16: two separate roundings (float64 ->
  // float32, then float32 -> bf16).  A (__bf16) cast of (float)(double)
  // could be folded into one conversion from float64, which is not the same
  // result; the conversion is therefore written in assembly.
  uint32_t y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] = cvt_pk_bf16((float)(xd[2 * i] * r), (float)(xd[2 * i + 1] * r));
  return make_uint4(y[0], y[1], y[2], y[3]);
}

// The same normalisation with a row held by an 8-lane group (lanes sharing
// lane/8), 16 consecutive elements per lane (x0: elements 0..7, x1: 8..15).
// Identical results: the sum is exact on the fast path (any order), the
// slow path rounds in the group's first lane, and the division is per
// element.

// Step 1: the elements as float64, their sum of squares, and whether that
// float64 sum is exact (the row's magnitudes span at most 15 binades).
__device__ __forceinline__ void row8_sum_sq(const uint4& x0, const uint4& x1, double* xd, double& s, bool& exact) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  const uint32_t w[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    xd[2 * i] = (double)bf16lo(w[i]);
    xd[2 * i + 1] = (double)bf16hi(w[i]);
  }
  u16x2 mx = {0, 0};
  u16x2 mn = {0xffff, 0xffff};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const u16x2 m = __builtin_bit_cast(u16x2, w[i] & 0x7fff7fffu);
    mx = __builtin_elementwise_max(mx, m);
    mn = __builtin_elementwise_min(mn, m - (u16x2){1, 1});
  }
  int emax = int(mx[0] > mx[1] ? mx[0] : mx[1]);
  int emin = int(mn[0] < mn[1] ? mn[0] : mn[1]) + 1;
  s = 0.0;
#pragma unroll
  for (int i = 0; i < 16; ++i) s = fma(xd[i], xd[i], s);
  s = row8_sum(s);
  emax = row8_max(emax) >> 7;
  emin = row8_min(emin) >> 7;
  exact = (emax == 0 && emin == 512) || (max(emax, 1) - max(emin, 1) <= 15);
}

// Slow path: the exact sum of squares in double-double, rounded once to
// float32 in the group's first lane and broadcast to the group.
__device__ __forceinline__ float row8_sum_sq_dd(const double* xd) {
  double hi = 0.0, lo = 0.0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    double t, e;
    two_sum(hi, xd[i] * xd[i], t, e);
    hi = t;
    lo += e;
  }
#pragma unroll
  for (int off = 1; off < 8; off <<= 1) {
    const double oh = __shfl_xor(hi, off, 64);
    const double ol = __shfl_xor(lo, off, 64);
    double t, e;
    two_sum(hi, oh, t, e);
    const double l = lo + ol + e;
    hi = t + l;
    lo = l - (hi - t);
  }
  return __shfl(dd_to_f32(hi, lo), (threadIdx.x & 63) & ~7, 64);
}

// Step 3: y = bf16(x / sqrt(s32 + 1e-6)), correctly rounded.
__device__ __forceinline__ void row8_scale(uint4& x0, uint4& x1, const double* xd, float s32) {
  const float t = s32 + 1e-6f;
  const float d = (float)__builtin_sqrt((double)t);
  const double r = 1.0 / (double)d;
  uint32_t y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = cvt_pk_bf16((float)(xd[2 * i] * r), (float)(xd[2 * i + 1] * r));
  x0 = make_uint4(y[0], y[1], y[2], y[3]);
  x1 = make_uint4(y[4], y[5], y[6], y[7]);
}

__device__ __forceinline__ void l2norm_row8(uint4& x0, uint4& x1) {
  double xd[16], s;
  bool exact;
  row8_sum_sq(x0, x1, xd, s, exact);
  float s32 = (float)s;
  if (!__all(exact)) {
    const float r = row8_sum_sq_dd(xd);
    if (!exact) s32 = r;
  }
  row8_scale(x0, x1, xd, s32);
}

}  // namespace kda
