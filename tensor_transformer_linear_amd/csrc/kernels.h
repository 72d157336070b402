// Host-side launch interfaces of the gfx950 kernels (internal to libtpshard).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tpshard.h"

namespace tpk {

// Output stage of the NT GEMM: y = round(act(acc + bias)), stored at a remapped column.
struct GemmEpilogue {
  const uint16_t* bias;  // bf16 [N] or nullptr
  void* C;               // bf16 or f32 output
  int64_t ldc;           // elements between output rows
  int act;               // TP_ACT_*
  int out_f32;           // 0: bf16 output, 1: f32 output
  int accumulate;        // f32 only: C += result (one rounding)
  int n_seg;             // column segments; 0 = output column is the local column
  int seg_end[TP_MAX_SUBPARAMS];    // exclusive local end column of each segment
  int seg_delta[TP_MAX_SUBPARAMS];  // output column minus local column inside the segment
  const float* row_scale;  // f32 [M] or nullptr: acc * row_scale[m] * col_scale[n] before the bias
  const float* col_scale;  // f32 [N] (with row_scale)
  // SwiGLU (glu = 1): output column c pairs its gate (B row of c) with its value (glu_off B rows
  // further) and stores bf16(swish(bf16(gate)) * bf16(value)); a tile then covers BN / 2 output
  // columns. bf16 output only; no bias, activation or scales.
  int glu;
  int glu_off;
  // Optional per-head output placement (c_head_w > 0, used with glu): column c of head
  // h = c / c_head_w goes to h * c_head_pitch + c_head_off + c % c_head_w.
  int c_head_w, c_head_pitch, c_head_off;
};

// C[M,N] = A[M,K] * B[N,K]^T with both operands K-contiguous (weights as stored).
struct GemmProblem {
  const uint16_t* A;  // bf16 [M, lda] (E4M3 bytes when fp8)
  int64_t lda;        // elements
  const uint16_t* B;  // bf16 [N, ldb] (E4M3 bytes when fp8)
  int64_t ldb;
  int fp8;            // 1: A and B are OCP E4M3 codes (direct-to-LDS path only, K % 64 == 0)
  int M, N, K;
  // Optional RMSNorm applied to A while it is staged: a' = bf16(bf16(a * row_r[m]) * col_t[k]),
  // or bf16(a * row_r[m]) when col_t is null.
  const float* row_r;     // f32 [M] or nullptr (no normalisation)
  const uint16_t* col_t;  // bf16 [K] or nullptr
  // Optional per-head B rows (b_head_w > 0): column c of head h = c / b_head_w reads B row
  // h * b_head_pitch + b_head_off + c % b_head_w (a slice of every head's rows).
  int b_head_w, b_head_pitch, b_head_off;
  GemmEpilogue ep;
};

// Tile configurations the launcher can pick (see gemm.hip for their shapes).
enum GemmTile : int {
  TILE_AUTO = -1,
  TILE_256x256 = 0,
  TILE_256x128 = 1,
  TILE_128x128 = 2,
  TILE_128x256 = 3,
  TILE_256x224 = 4,
  TILE_128x64 = 5,
  TILE_64x64 = 6,
  TILE_COUNT = 7
};

// Main-loop path: automatic (direct-to-LDS when there is no A transform and K % 32 == 0,
// else register staging), or forced for testing.
enum GemmPath : int { GEMM_PATH_AUTO = -1, GEMM_PATH_REGISTER = 0, GEMM_PATH_DMA = 1 };

hipError_t launch_gemm(const GemmProblem& p, int tile, int path, hipStream_t stream);
int gemm_pick_tile(int M, int N, int K);
// E4M3 x E4M3 GEMM (p.fp8 = 1) on the fp8 matrix cores; tile: TILE_AUTO, TILE_256x256 or TILE_128x128.
hipError_t launch_gemm_fp8(const GemmProblem& p, int tile, hipStream_t stream);
int gemm_fp8_pick_tile(int M, int N, int K);

// Per-row E4M3 quantisation of bf16 activations: scale[m] = amax/448 (1 for a zero row),
// q = nearest E4M3 code of x / scale (ties to even, saturating, signed zero). K % 8 == 0.
hipError_t launch_quantize_rows_e4m3(const uint16_t* x, int M, int K, uint8_t* q, float* scale, hipStream_t stream);

// One rank's embedding rows: out[t] = table[tokens[t] - off] when the id falls in the shard
// [off, off + rows) and in [0, vocab), else zeros. E % 8 == 0.
hipError_t launch_embed_shard(const int32_t* tokens, int n, int vocab, int rows, int off, const uint16_t* table,
                              int E, uint16_t* out, hipStream_t stream);

// One destination rank's sequence-parallel reduce-scatter of the ranks' float32 partials
// [batch * seq, N]: for output row i = b * sl + t (source row b * seq + dest * sl + t),
// S = rank-ordered float32 sum; y_sum = S and/or z = bf16(S + residual) (residual may be null).
// N % 4 == 0; every pointer 16-byte aligned.
struct ReduceScatterProblem {
  const float* part[TP_MAX_RANKS];
  int tp, dest;
  int64_t seq, sl, N;
  int64_t chunks;  // output rows * N / 4
  const uint16_t* residual;
  uint16_t* z;
  float* y_sum;
};
hipError_t launch_reduce_scatter(const ReduceScatterProblem& p, hipStream_t stream);

// RMSNorm statistics: r[m] = rsqrt(mean_k x^2 + eps) for every row, t[k] = bf16(1 + s[k]),
// and, when xnorm is non-null, the normalised bf16 rows.
hipError_t launch_rmsnorm_rows(const uint16_t* x, int M, int K, const uint16_t* scale, float eps, float* r,
                               uint16_t* t, uint16_t* xnorm, hipStream_t stream);

struct LmHeadProblem {
  const uint16_t* x;     // bf16 [B, K]
  const void* w;         // bf16 or e4m3 [V, K]
  const float* wscale;   // f32 [V, K/128] (fp8) or nullptr
  int w_fp8;
  int B, K, V;
  int chunk;             // rows per chunk (last chunk takes the remainder)
  float* logits;         // f32 [B, V]
  int32_t* argmax;       // int32 [B]
  float* maxval;         // f32 [B] or nullptr
  void* workspace;
};
size_t lm_head_workspace_bytes(int V);  // the largest need over the launch shapes and chunk sizes
// The workspace one launch shape needs (-1: the default shape).
size_t lm_head_shape_workspace_bytes(int shape, int B, int V, int K, bool fp8, int chunk);
// This GPU's device scratch for the allocation-free entry point (its address, found once per
// device with the device current) and its size.
hipError_t lm_head_scratch(void** ptr, size_t* bytes);
int lm_head_shape_count();
// shape: -1 = default launch shape, else an index into the LM head's shape table (tuning).
hipError_t launch_lm_head(const LmHeadProblem& p, int shape, hipStream_t stream);

}  // namespace tpk
