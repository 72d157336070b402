// K2 (row statistics): RMSNorm prologue of the column GEMM.
//
// [palm] allgather_layernorm: statistics in float32, r = rsqrt(mean(x^2) + eps),
// n = bf16(x * r); with a learned scale, t = bf16(1 + s) and y = bf16(n * t).
//
// One workgroup per row. Each thread sums the squares of its 16-byte chunks of the
// row in float64 (squares of bf16 values are exact, and so are their sums while the
// row's nonzero values span less than about 2^12: 16 significant bits, twice the
// span and 13 bits of count against float64's 53; no finite bf16 value overflows);
// the partial sums are combined in float64 and r is rounded to float32 once. The row is read once
// from HBM (non-temporal loads for the chunks held in registers: 180 -> 175 us on a
// 32768 x 8192 pass; non-temporal stores of the normalised rows, which the GEMM reads
// next, measured slower); when the normalised row is requested it is produced in the
// same pass from registers (rows up to 8192 wide) or from a second, cache-resident read.
// Workgroup 0 also writes t = bf16(1 + s), which the GEMM applies while staging A.
#include "common.h"
#include "kernels.h"

namespace tpk {

namespace {

constexpr int RMS_THREADS = 256;
constexpr int RMS_HELD = 4;  // 16-byte chunks per thread kept in registers (8192 bf16 per row)

__global__ __launch_bounds__(RMS_THREADS) void rmsnorm_rows_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                                   const uint16_t* __restrict__ scale, double eps,
                                                                   float* __restrict__ r_out,
                                                                   uint16_t* __restrict__ t_out,
                                                                   uint16_t* __restrict__ xnorm) {
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int nchunk = K / 8;
  const uint16_t* xr = x + (int64_t)row * K;

  if (row == 0 && t_out != nullptr && scale != nullptr) {
    for (int k = tid; k < K; k += RMS_THREADS) t_out[k] = f32_to_bf16(1.0f + bf16_to_f32(scale[k]));
  }

  u32x4_t held[RMS_HELD];
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < RMS_HELD; ++i) {
    int c = tid + i * RMS_THREADS;
    if (c < nchunk) {
      held[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(xr + c * 8));
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const double lo = bf16_lo(held[i][w]), hi = bf16_hi(held[i][w]);
        ss = fma(lo, lo, ss);
        ss = fma(hi, hi, ss);
      }
    }
  }
  for (int c = tid + RMS_HELD * RMS_THREADS; c < nchunk; c += RMS_THREADS) {
    u32x4_t v = *reinterpret_cast<const u32x4_t*>(xr + c * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const double lo = bf16_lo(v[w]), hi = bf16_hi(v[w]);
      ss = fma(lo, lo, ss);
      ss = fma(hi, hi, ss);
    }
  }

  // Combine the 256 partial sums: wave reduction, then across the four waves.
  double d = ss;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) d += __shfl_xor(d, off, 64);
  __shared__ double wsum[RMS_THREADS / 64];
  __shared__ float r_sh;
  if ((tid & 63) == 0) wsum[tid >> 6] = d;
  __syncthreads();
  if (tid == 0) {
    double tot = 0.0;
    for (int w = 0; w < RMS_THREADS / 64; ++w) tot += wsum[w];
    float r = (float)(1.0 / sqrt(tot / (double)K + eps));
    r_sh = r;
    if (r_out != nullptr) r_out[row] = r;
  }
  __syncthreads();
  if (xnorm == nullptr) return;

  const float r = r_sh;
  uint16_t* yr = xnorm + (int64_t)row * K;
  auto emit = [&](int c, u32x4_t v) {
    u32x4_t o;
    if (scale != nullptr) {
      const u32x4_t s = *reinterpret_cast<const u32x4_t*>(scale + c * 8);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t n = pack_bf16x2(bf16_lo(v[w]) * r, bf16_hi(v[w]) * r);
        uint32_t t = pack_bf16x2(1.0f + bf16_lo(s[w]), 1.0f + bf16_hi(s[w]));
        o[w] = pack_bf16x2(bf16_lo(n) * bf16_lo(t), bf16_hi(n) * bf16_hi(t));
      }
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) o[w] = pack_bf16x2(bf16_lo(v[w]) * r, bf16_hi(v[w]) * r);
    }
    *reinterpret_cast<u32x4_t*>(yr + c * 8) = o;
  };
#pragma unroll
  for (int i = 0; i < RMS_HELD; ++i) {
    int c = tid + i * RMS_THREADS;
    if (c < nchunk) emit(c, held[i]);
  }
  for (int c = tid + RMS_HELD * RMS_THREADS; c < nchunk; c += RMS_THREADS)
    emit(c, *reinterpret_cast<const u32x4_t*>(xr + c * 8));
}

}  // namespace

hipError_t launch_rmsnorm_rows(const uint16_t* x, int M, int K, const uint16_t* scale, float eps, float* r,
                               uint16_t* t, uint16_t* xnorm, hipStream_t stream) {
  hipLaunchKernelGGL(rmsnorm_rows_kernel, dim3(M), dim3(RMS_THREADS), 0, stream, x, M, K, scale, (double)eps, r, t,
                     xnorm);
  return hipGetLastError();
}

}  // namespace tpk
