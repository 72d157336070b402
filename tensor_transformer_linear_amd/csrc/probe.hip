// Rounding of the two matrix instructions the GEMMs use, observed on fixed operands (tuning
// library only; a test pins the accumulation model that the parity tests' error bounds rest on).
//
// One wave runs one instruction with A = 32 test rows, B = all ones and C = one value per row,
// so output (i, j) = C[i] + the sum of row i's products (A[i, k] * 1):
//  * v_mfma_f32_32x32x16_bf16: A [32][16] bf16, lane l holds row l % 32, K 8 (l / 32) .. +8;
//  * v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3, unit scales): A [32][64] E4M3, lane l holds row
//    l % 32, K 32 (l / 32) .. +32.
// The accumulator layout: lane l holds column l % 32 and rows 8 (v / 4) + 4 (l / 32) + v % 4.
#include <string.h>

#include "common.h"
#include "tpshard_tuning.h"

namespace {

typedef __attribute__((ext_vector_type(8))) int i32x8_t;

template <bool FP8>
__global__ __launch_bounds__(64) void mfma_row_sums_kernel(const unsigned char* a, const float* c, float* out) {
  const int l = threadIdx.x, row = l % 32;
  f32x16_t acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = c[8 * (v / 4) + 4 * (l / 32) + v % 4];
  if constexpr (FP8) {
    uint32_t av[8], bv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      av[i] = *reinterpret_cast<const uint32_t*>(a + row * 64 + 32 * (l / 32) + 4 * i);
      bv[i] = 0x38383838u;  // E4M3 1.0
    }
    i32x8_t A, B;
    memcpy(&A, av, 32);
    memcpy(&B, bv, 32);
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc, 0, 0, 0, 0, 0, 0);
  } else {
    const u32x4_t av = *reinterpret_cast<const u32x4_t*>(a + (row * 16 + 8 * (l / 32)) * 2);
    const u32x4_t bv = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, bv),
                                                  acc, 0, 0, 0);
  }
  if (l % 32 == 0) {
#pragma unroll
    for (int v = 0; v < 16; ++v) out[8 * (v / 4) + 4 * (l / 32) + v % 4] = acc[v];
  }
}

}  // namespace

extern "C" TP_API int tpt_mfma_row_sums(int fp8, const void* a, const float* c, float* out, void* stream) {
  if (a == nullptr || c == nullptr || out == nullptr) return TP_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(a) & 15) || (reinterpret_cast<uintptr_t>(c) & 3) ||
      (reinterpret_cast<uintptr_t>(out) & 3))
    return TP_ERR_UNSUPPORTED;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (fp8)
    hipLaunchKernelGGL(mfma_row_sums_kernel<true>, dim3(1), dim3(64), 0, s, static_cast<const unsigned char*>(a), c,
                       out);
  else
    hipLaunchKernelGGL(mfma_row_sums_kernel<false>, dim3(1), dim3(64), 0, s, static_cast<const unsigned char*>(a), c,
                       out);
  return hipGetLastError() == hipSuccess ? TP_OK : TP_ERR_HIP;
}
