// Device helpers shared by the gfx950 kernels of the TP linear hot path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "tpshard.h"

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;   // one MFMA bf16 operand (8 K-values per lane)
typedef __attribute__((ext_vector_type(16))) float f32x16_t;   // 32x32 MFMA accumulator slice per lane
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;  // 16 bytes moved as one vector

namespace tpk {

// bf16 <-> f32. A bf16 value is the high half of a float32 pattern, so widening
// is a shift; narrowing uses gfx950's v_cvt_pk_bf16_f32 (round to nearest even).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

// exp(y) for finite y in float32: y log2 e is split into h + l (log2 e as two floats, the
// product's error from an fma) and 2^(h + l) = 2^h (1 + l ln 2), with the hardware exp2 for 2^h,
// so the rounding of y log2 e is not amplified for large |y|.
__device__ __forceinline__ float exp_split(float y) {
  constexpr float kL2eHi = 1.44269502162933349609375f;  // log2 e, leading float
  constexpr float kL2eLo = 1.92596299e-8f;               // log2 e - kL2eHi
  const float h = y * kL2eHi;
  const float l = fmaf(y, kL2eLo, fmaf(y, kL2eHi, -h));  // y log2 e = h + l
  const float e2 = __builtin_amdgcn_exp2f(h);
  return fmaf(e2, l * 0.69314718055994531f, e2);
}

// Exact (erf) GELU in float32: 0.5 a (1 + erf(a / sqrt 2)), evaluated as 0.5 a erfc(-a / sqrt 2)
// (the same function) so that large negative inputs keep their relative accuracy instead of
// cancelling in 1 + erf. erfc(z), z = |a| / sqrt 2, is the Chebyshev-fitted approximation erfcc
// of Press et al., Numerical Recipes (t = 1 / (1 + z / 2), erfc(z) = t exp(-z^2 + P(t)) with a
// degree-9 polynomial P; fractional error below 1.2e-7 for every z >= 0), and erfc(-z) =
// 2 - erfc(z) for a > 0. Two steps keep float32 evaluation close to that bound:
// - the exponent takes z^2 as a^2 / 2 from the exact split a^2 = s + e (s rounded, e = fma(a, a,
//   -s)), so the rounding of a / sqrt 2 is not amplified by exp;
// - exp(y) from exp_split.
// z stops at 13, where erfc underflows float32 (larger |a| would overflow the square).
// Measured against float64 erf-GELU in a float32 emulation of these steps, every finite bf16
// input rounds to the same bf16 output; the largest errors are about 6 float32 ulps for
// |a| < 1 and 2 for a > 1 (tens of ulps in the negative tail below -3, where |GELU| < 0.005).
__device__ __forceinline__ float gelu_erf(float a) {
  const float ab = fabsf(a);
  const float z = fminf(ab * 0.70710678118654752f, 13.0f);
  const float d = fmaf(0.5f, z, 1.0f);
  float t = __builtin_amdgcn_rcpf(d);
  t = fmaf(t, fmaf(-d, t, 1.0f), t);  // one Newton step on the reciprocal
  float p = 0.17087277f;
  p = fmaf(p, t, -0.82215223f);
  p = fmaf(p, t, 1.48851587f);
  p = fmaf(p, t, -1.13520398f);
  p = fmaf(p, t, 0.27886807f);
  p = fmaf(p, t, -0.18628806f);
  p = fmaf(p, t, 0.09678418f);
  p = fmaf(p, t, 0.37409196f);
  p = fmaf(p, t, 1.00002368f);
  p = fmaf(p, t, -1.26551223f);
  const float ac = fminf(ab, 18.0f);
  const float sq = ac * ac;
  const float sq_err = fmaf(ac, ac, -sq);  // a^2 = sq + sq_err exactly
  const float y = fmaf(-0.5f, sq_err, fmaf(-0.5f, sq, p));
  const float q = t * exp_split(y);  // erfc(z)
  return 0.5f * a * (a < 0.0f ? q : 2.0f - q);
}

// SwiGLU of one output from float32 accumulators: the gate and the value are rounded to bf16
// first, then Swish with unit slope, g / (1 + exp(-g)), times the value, in float32. For very
// negative g the Swish underflows (a subnormal, or -0 below about -104), as float64 rounded to
// float32 does.
__device__ __forceinline__ float swiglu_of(float gate, float value) {
  const float g = bf16_to_f32(f32_to_bf16(gate)), u = bf16_to_f32(f32_to_bf16(value));
  // swish(g) = g / (1 + exp(-g)) from E = exp(-|g|) in (0, 1], so nothing overflows: g / (1 + E)
  // for g >= 0, g E / (1 + E) for g < 0 (E is exactly 0 below -150, where -inf gives NaN as
  // -inf / (1 + inf) does). The reciprocal of 1 + E, in (1, 2], is the hardware estimate plus one
  // Newton step. In a float32 emulation the Swish of every finite bf16 gate is within 2.3 ulp of
  // float64 (the correctly rounded library exp and divide: 1.8).
  const float e = exp_split(fmaxf(-fabsf(g), -150.0f));
  const float d = 1.0f + e;
  float r = __builtin_amdgcn_rcpf(d);
  r = fmaf(r, fmaf(-d, r, 1.0f), r);
  return (g < 0.0f ? (g * e) * r : g * r) * u;
}

// Compile-time loop: f(std::integral_constant<int, 0>) ... f(<N-1>). Register arrays indexed
// by these constants stay in registers whatever the unroller decides.
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Number of XCDs of an MI355X; consecutive workgroup ids are dispatched round-robin over them.
constexpr int kNumXcd = 8;

// Map a hardware workgroup id to a logical tile id so that logical ids that are
// close together run on the same XCD (and share its L2): the ids that land on
// XCD x (bid % 8 == x) become one contiguous logical range.
__device__ __forceinline__ int xcd_remap(int bid, int nb) {
  int xcd = bid % kNumXcd, slot = bid / kNumXcd;
  int per = nb / kNumXcd, rem = nb % kNumXcd;
  return xcd * per + (xcd < rem ? xcd : rem) + slot;
}

}  // namespace tpk
