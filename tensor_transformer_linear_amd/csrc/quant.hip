// Per-row (per-token) E4M3 quantisation of bf16 activations, for the fp8 prefill GEMM.
//
// [palm] transformer_layer_weight_gathered: a QuantizedLayer multiplies by quantised weights
// and applies the per-output-channel scale after the matmul. To run that product on fp8
// matrix cores the activations are quantised too, one float32 scale per row:
// s = amax|x| / 448 (1 for an all-zero row), q = e4m3(x / s). Both divisions are IEEE float32
// divisions (round to nearest even), and the E4M3 code is the nearest one, ties to the even
// mantissa, saturating at 448, with the float's sign bit (E4M3 has a signed zero).
//
// One workgroup per row. Rows up to 8192 wide stay in registers between the amax pass and
// the encoding pass, so x is read once; wider rows are read a second time (from cache).
//
// Rows with a finite maximum encode with gfx950's packed float32 -> E4M3 conversion (two codes
// per instruction), after clamping the quotient to +-448: on every finite value up to 464 in
// magnitude that conversion rounds exactly as the definition above (nearest, ties to the even
// mantissa, subnormal codes, signed zero), and the clamp gives the saturated code beyond. Rows
// holding an infinity or NaN keep the integer encoder below (every such value saturates).

#include "common.h"
#include "kernels.h"

namespace tpk {

namespace {

constexpr int Q_THREADS = 256;
constexpr int Q_HELD = 4;  // 16-byte chunks per thread kept in registers (8192 bf16 per row)

// Nearest E4M3 code of a float32, written from the format's definition: normal codes carry
// three mantissa bits (round the float's 23 to 3, nearest even; a carry bumps the exponent),
// codes below 2^-6 are multiples of 2^-9 (exact scaling by 512, then nearest even to an
// integer 0..8, where 8 is the first normal code), 448 and beyond saturate to 0x7E.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a >= 0x43E00000u) {  // |v| >= 448
    code = 0x7Eu;
  } else if (a < 0x3C800000u) {  // |v| < 2^-6
    code = (uint32_t)__float2int_rn(__uint_as_float(a) * 512.0f);
  } else {
    int e = (int)(a >> 23) - 127;  // -6 .. 8
    const uint32_t m = a & 0x7FFFFFu;
    uint32_t r = m >> 20;
    const uint32_t rest = m & 0xFFFFFu;
    if (rest > 0x80000u || (rest == 0x80000u && (r & 1u))) ++r;
    if (r == 8u) {
      r = 0u;
      ++e;
    }
    code = ((uint32_t)(e + 7) << 3) | r;
  }
  return sign | code;
}

typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

// The row is read once and its codes are written once: non-temporal loads and stores
// (145 -> 134 us at 32768 x 8192).
__global__ __launch_bounds__(Q_THREADS) void quantize_rows_e4m3_kernel(const uint16_t* __restrict__ x, int K,
                                                                      uint8_t* __restrict__ q,
                                                                      float* __restrict__ scale) {
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int nchunk = K / 8;
  const uint16_t* xr = x + (int64_t)row * K;
  uint8_t* qr = q + (int64_t)row * K;

  // pass 1: the row's largest magnitude (exact: the maximum of bf16 values)
  u32x4_t held[Q_HELD];
  uint32_t amax_bits = 0;  // |x| as float bits: non-negative floats order like their bits
  auto fold = [&](const u32x4_t& c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      amax_bits = max(amax_bits, (c[i] << 16) & 0x7FFFFFFFu);
      amax_bits = max(amax_bits, c[i] & 0x7FFF0000u);
    }
  };
#pragma unroll
  for (int i = 0; i < Q_HELD; ++i) {
    const int c = tid + i * Q_THREADS;
    if (c < nchunk) {
      held[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(xr + c * 8));  // read once
      fold(held[i]);
    }
  }
  for (int c = tid + Q_HELD * Q_THREADS; c < nchunk; c += Q_THREADS)
    fold(*reinterpret_cast<const u32x4_t*>(xr + c * 8));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax_bits = max(amax_bits, (uint32_t)__shfl_xor((int)amax_bits, off, 64));
  __shared__ uint32_t wmax[Q_THREADS / 64];
  if ((tid & 63) == 0) wmax[tid >> 6] = amax_bits;
  __syncthreads();
  uint32_t m = wmax[0];
#pragma unroll
  for (int w = 1; w < Q_THREADS / 64; ++w) m = max(m, wmax[w]);
  const float amax = __uint_as_float(m);
  const float s = amax == 0.0f ? 1.0f : __fdiv_rn(amax, 448.0f);
  if (tid == 0) scale[row] = s;

  // pass 2: codes, eight per 8-byte store
  const bool finite_row = m < 0x7F800000u;
  auto encode = [&](const u32x4_t& c, int chunk) {
    if (finite_row) {
      float y[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        y[2 * i] = __fdiv_rn(__uint_as_float(c[i] << 16), s);
        y[2 * i + 1] = __fdiv_rn(__uint_as_float(c[i] & 0xFFFF0000u), s);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = __builtin_amdgcn_fmed3f(y[e], -448.0f, 448.0f);
      uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
      uint32_t hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
      __builtin_nontemporal_store(u32x2_t{lo, hi}, reinterpret_cast<u32x2_t*>(qr + chunk * 8));
      return;
    }
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t c0 = e4m3_code(__fdiv_rn(__uint_as_float(c[i] << 16), s));
      const uint32_t c1 = e4m3_code(__fdiv_rn(__uint_as_float(c[i] & 0xFFFF0000u), s));
      const uint32_t pair = c0 | (c1 << 8);
      if (i < 2)
        lo |= pair << (16 * i);
      else
        hi |= pair << (16 * (i - 2));
    }
    *reinterpret_cast<uint2*>(qr + chunk * 8) = make_uint2(lo, hi);
  };
#pragma unroll
  for (int i = 0; i < Q_HELD; ++i) {
    const int c = tid + i * Q_THREADS;
    if (c < nchunk) encode(held[i], c);
  }
  for (int c = tid + Q_HELD * Q_THREADS; c < nchunk; c += Q_THREADS)
    encode(*reinterpret_cast<const u32x4_t*>(xr + c * 8), c);
}

}  // namespace

hipError_t launch_quantize_rows_e4m3(const uint16_t* x, int M, int K, uint8_t* q, float* scale, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_rows_e4m3_kernel, dim3(M), dim3(Q_THREADS), 0, stream, x, K, q, scale);
  return hipGetLastError();
}

}  // namespace tpk
