// Sequence-parallel reduce-scatter of row-parallel partials with the residual add, emulated on
// one GPU for one destination rank.
//
// [nanotron] MLP Module: the row-parallel c_proj hands each rank [batch, seq / tp, hidden];
// [palm] reduce-scatters the o_wo partials and adds the residual, z = bf16(y_out + x). Rank d
// keeps positions [d sl, (d + 1) sl) of every sequence (sl = seq / tp). Its rows sum the
// ranks' float32 partials in rank order, S = ((P_0 + P_1) + P_2) + ..., each addition rounded
// to float32; the residual is added in float32 and the result rounded once to bf16.
//
// Memory-bound: each thread owns four consecutive columns of one output row, issues the tp
// 16-byte partial loads together, then adds them in rank order.
#include "common.h"
#include "kernels.h"

namespace tpk {

namespace {

constexpr int RS_THREADS = 256;

// TPC > 0: the rank count is a compile-time constant (loads unrolled); 0: runtime loop. Each
// partial element is read exactly once: non-temporal loads (26.0 -> 23.9 us per destination
// on the llama-8B MLP shard).
template <int TPC>
__global__ __launch_bounds__(RS_THREADS) void reduce_scatter_kernel(ReduceScatterProblem p) {
  const int64_t id = (int64_t)blockIdx.x * RS_THREADS + threadIdx.x;
  if (id >= p.chunks) return;
  const int64_t n4 = p.N / 4;
  const int64_t i = id / n4;  // output row: token t of sequence b in the slice
  const int64_t c = (id - i * n4) * 4;
  const int64_t b = i / p.sl, t = i - b * p.sl;
  const int64_t src = (b * p.seq + (int64_t)p.dest * p.sl + t) * p.N + c;
  f32x4_t s;
  if constexpr (TPC > 0) {
    f32x4_t v[TPC];
#pragma unroll
    for (int r = 0; r < TPC; ++r) v[r] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p.part[r] + src));
    s = v[0];
#pragma unroll
    for (int r = 1; r < TPC; ++r) s += v[r];
  } else {
    s = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p.part[0] + src));
    for (int r = 1; r < p.tp; ++r) s += __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p.part[r] + src));
  }
  const int64_t o = i * p.N + c;
  if (p.y_sum != nullptr) *reinterpret_cast<f32x4_t*>(p.y_sum + o) = s;
  if (p.z != nullptr) {
    if (p.residual != nullptr) {
      const uint2 x = *reinterpret_cast<const uint2*>(p.residual + o);
      s[0] += bf16_lo(x.x);
      s[1] += bf16_hi(x.x);
      s[2] += bf16_lo(x.y);
      s[3] += bf16_hi(x.y);
    }
    uint2 pk;
    pk.x = pack_bf16x2(s[0], s[1]);
    pk.y = pack_bf16x2(s[2], s[3]);
    *reinterpret_cast<uint2*>(p.z + o) = pk;
  }
}

}  // namespace

hipError_t launch_reduce_scatter(const ReduceScatterProblem& p, hipStream_t stream) {
  if (p.chunks == 0) return hipSuccess;
  const dim3 grid((unsigned)((p.chunks + RS_THREADS - 1) / RS_THREADS)), block(RS_THREADS);
  switch (p.tp) {
    case 1: hipLaunchKernelGGL(reduce_scatter_kernel<1>, grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL(reduce_scatter_kernel<2>, grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL(reduce_scatter_kernel<4>, grid, block, 0, stream, p); break;
    case 8: hipLaunchKernelGGL(reduce_scatter_kernel<8>, grid, block, 0, stream, p); break;
    case 16: hipLaunchKernelGGL(reduce_scatter_kernel<16>, grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL(reduce_scatter_kernel<0>, grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}

}  // namespace tpk
