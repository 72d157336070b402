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

// Exact (erf) GELU in float32: 0.5 a (1 + erf(a / sqrt 2)), evaluated as 0.5 a erfc(-a / sqrt 2)
// (the same function) so that large negative inputs keep their relative accuracy instead of
// cancelling in 1 + erf.
__device__ __forceinline__ float gelu_erf(float a) { return 0.5f * a * erfcf(-a * 0.70710678118654752f); }

// SwiGLU of one output from float32 accumulators: the gate and the value are rounded to bf16
// first, then Swish with unit slope, g / (1 + exp(-g)), times the value, in float32. For
// g < -88.7 exp(-g) is inf and the Swish is -0, its limit.
__device__ __forceinline__ float swiglu_of(float gate, float value) {
  const float g = bf16_to_f32(f32_to_bf16(gate)), u = bf16_to_f32(f32_to_bf16(value));
  return g / (1.0f + expf(-g)) * u;
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
