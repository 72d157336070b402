// Tuning library entry points (tpshard_tuning.h): the product entry points' bodies with
// the launch choices passed in. Linked only into libtpshard_tuning.so.
#include <limits.h>

#include "abi_impl.h"
#include "tpshard_tuning.h"

namespace {

tpabi::Tuning make(int tile, int path, int lm_shape) {
  tpabi::Tuning t;
  t.tile = tile;
  t.path = path;
  t.lm_shape = lm_shape;
  return t;
}

}  // namespace

extern "C" {

TP_API int tpt_column_linear(const void* x, int64_t M, int64_t K, const void* w_shard, const void* bias_shard,
                             const int64_t* subparam_sizes, int n_sub, int tp_size, int rank, int act, void* y,
                             int y_dtype, int layout, int64_t ldy, void* stream, int tile, int path) {
  const tpabi::Tuning t = make(tile, path, -1);
  if (int st = tpabi::check_tuning(t)) return st;
  return tpabi::column_linear(x, M, K, w_shard, bias_shard, subparam_sizes, n_sub, tp_size, rank, act, y, y_dtype,
                              layout, ldy, stream, t);
}

TP_API int tpt_column_linear_fp8(const void* x_q, const float* x_scale, int64_t M, int64_t K, const void* w_q,
                                 const float* w_scale, const void* bias_shard, const int64_t* subparam_sizes,
                                 int n_sub, int tp_size, int rank, int act, void* y, int y_dtype, int layout,
                                 int64_t ldy, void* stream, int tile) {
  const tpabi::Tuning t = make(tile, -1, -1);
  if (int st = tpabi::check_tuning(t)) return st;
  return tpabi::column_linear_fp8(x_q, x_scale, M, K, w_q, w_scale, bias_shard, subparam_sizes, n_sub, tp_size, rank,
                                  act, y, y_dtype, layout, ldy, stream, t);
}

TP_API int tpt_row_linear_partial(const void* x_shard, int64_t M, int64_t K_logical, int64_t N, const void* w_shard,
                                  const void* bias, int tp_size, int rank, float* y_partial, int accumulate,
                                  void* stream, int tile, int path) {
  const tpabi::Tuning t = make(tile, path, -1);
  if (int st = tpabi::check_tuning(t)) return st;
  return tpabi::row_linear_partial(x_shard, M, K_logical, N, w_shard, bias, tp_size, rank, y_partial, accumulate,
                                   stream, t);
}

TP_API int tpt_qwi_swiglu(const void* xnorm, int64_t M, int64_t E, int64_t heads, int64_t padded_heads, int64_t qkv,
                          int64_t ff, int tp_size, int rank, const void* w_qwi, void* q, void* y_fused, void* stream,
                          int tile, int path) {
  const tpabi::Tuning t = make(tile, path, -1);
  if (int st = tpabi::check_tuning(t)) return st;
  return tpabi::qwi_swiglu(xnorm, M, E, heads, padded_heads, qkv, ff, tp_size, rank, w_qwi, q, y_fused, stream, t);
}

TP_API int tpt_o_wo_partial(const void* y_fused, int64_t M, int64_t heads, int64_t padded_heads, int64_t qkv,
                            int64_t ff, int64_t E, int tp_size, int rank, const void* w_o, float* y_partial,
                            int accumulate, void* stream, int tile, int path) {
  const tpabi::Tuning t = make(tile, path, -1);
  if (int st = tpabi::check_tuning(t)) return st;
  return tpabi::o_wo_partial(y_fused, M, heads, padded_heads, qkv, ff, E, tp_size, rank, w_o, y_partial, accumulate,
                             stream, t);
}

TP_API int tpt_rmsnorm_column_linear(const void* x, int64_t M, int64_t K, const void* scale, float eps,
                                     void* xnorm_out, const void* w_shard, const void* bias_shard,
                                     const int64_t* subparam_sizes, int n_sub, int tp_size, int rank, void* y,
                                     int y_dtype, int layout, int64_t ldy, void* workspace, size_t workspace_bytes,
                                     void* stream, int tile, int path) {
  const tpabi::Tuning t = make(tile, path, -1);
  if (int st = tpabi::check_tuning(t)) return st;
  return tpabi::rmsnorm_column_linear(x, M, K, scale, eps, xnorm_out, w_shard, bias_shard, subparam_sizes, n_sub,
                                      tp_size, rank, y, y_dtype, layout, ldy, workspace, workspace_bytes, stream, t);
}

TP_API int tpt_rmsnorm_rows(const void* x, int64_t M, int64_t K, const void* scale, float eps, void* xnorm_out,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return tpabi::rmsnorm_rows(x, M, K, scale, eps, xnorm_out, workspace, workspace_bytes, stream);
}

TP_API int tpt_lm_head_shard_argmax(const void* x, int64_t B, int64_t K, int64_t vocab, int tp_size, int rank,
                                    int64_t max_rows_per_chunk, const void* w_shard, int w_dtype,
                                    const float* w_block_scale, float* logits, int32_t* argmax_local,
                                    float* max_logit, void* workspace, size_t workspace_bytes, void* stream,
                                    int lm_shape) {
  const tpabi::Tuning t = make(-1, -1, lm_shape);
  if (int st = tpabi::check_tuning(t)) return st;
  return tpabi::lm_head_shard_argmax(x, B, K, vocab, tp_size, rank, max_rows_per_chunk, w_shard, w_dtype,
                                     w_block_scale, logits, argmax_local, max_logit, workspace, workspace_bytes,
                                     stream, t);
}

TP_API int tpt_gemm_pick_tile(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 1 || M > INT_MAX || N > INT_MAX || K > INT_MAX) return -1;
  return tpk::gemm_pick_tile((int)M, (int)N, (int)K);
}

TP_API int tpt_gemm_fp8_pick_tile(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 1 || M > INT_MAX || N > INT_MAX || K > INT_MAX) return -1;
  return tpk::gemm_fp8_pick_tile((int)M, (int)N, (int)K);
}

TP_API int tpt_lm_head_shape_count(void) { return tpk::lm_head_shape_count(); }

}  // extern "C"
