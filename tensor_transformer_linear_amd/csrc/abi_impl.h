// Internal entry points of libtpshard behind the exported C ABI (tpshard.h).
//
// Each function below is the body of the exported call of the same name (without the
// "tp_" prefix) with one more argument: the launch choices. The exported calls pass
// Tuning{} (every choice automatic), so the product library holds no mutable state
// besides the thread-local error message. The tuning library (tuning_abi.hip) exports
// variants that take the choices as explicit arguments, for tests and measurements.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "kernels.h"

namespace tpabi {

// Launch choices: tpk::TILE_AUTO or a tpk::GemmTile; tpk::GEMM_PATH_*; -1 or an LM-head
// launch shape index.
struct Tuning {
  int tile = tpk::TILE_AUTO;
  int path = tpk::GEMM_PATH_AUTO;
  int lm_shape = -1;
};

int column_linear(const void* x, int64_t M, int64_t K, const void* w_shard, const void* bias_shard,
                  const int64_t* subparam_sizes, int n_sub, int tp_size, int rank, int act, void* y, int y_dtype,
                  int layout, int64_t ldy, void* stream, const Tuning& tune);
int column_linear_fp8(const void* x_q, const float* x_scale, int64_t M, int64_t K, const void* w_q,
                      const float* w_scale, const void* bias_shard, const int64_t* subparam_sizes, int n_sub,
                      int tp_size, int rank, int act, void* y, int y_dtype, int layout, int64_t ldy, void* stream,
                      const Tuning& tune);
int row_linear_partial(const void* x_shard, int64_t M, int64_t K_logical, int64_t N, const void* w_shard,
                       const void* bias, int tp_size, int rank, float* y_partial, int accumulate, void* stream,
                       const Tuning& tune);
int qwi_swiglu(const void* xnorm, int64_t M, int64_t E, int64_t heads, int64_t padded_heads, int64_t qkv, int64_t ff,
               int tp_size, int rank, const void* w_qwi, void* q, void* y_fused, void* stream, const Tuning& tune);
int o_wo_partial(const void* y_fused, int64_t M, int64_t heads, int64_t padded_heads, int64_t qkv, int64_t ff,
                 int64_t E, int tp_size, int rank, const void* w_o, float* y_partial, int accumulate, void* stream,
                 const Tuning& tune);
int rmsnorm_column_linear(const void* x, int64_t M, int64_t K, const void* scale, float eps, void* xnorm_out,
                          const void* w_shard, const void* bias_shard, const int64_t* subparam_sizes, int n_sub,
                          int tp_size, int rank, void* y, int y_dtype, int layout, int64_t ldy, void* workspace,
                          size_t workspace_bytes, void* stream, const Tuning& tune);
int lm_head_shard_argmax(const void* x, int64_t B, int64_t K, int64_t vocab, int tp_size, int rank,
                         int64_t max_rows_per_chunk, const void* w_shard, int w_dtype, const float* w_block_scale,
                         float* logits, int32_t* argmax_local, float* max_logit, void* workspace,
                         size_t workspace_bytes, void* stream, const Tuning& tune);

// The RMSNorm pass of rmsnorm_column_linear alone: r and t into the workspace, the normalised
// rows into xnorm_out (which must be non-NULL).
int rmsnorm_rows(const void* x, int64_t M, int64_t K, const void* scale, float eps, void* xnorm_out, void* workspace,
                 size_t workspace_bytes, void* stream);

// Validates a tuning choice; sets the calling thread's message and returns a status.
int check_tuning(const Tuning& tune);

}  // namespace tpabi
