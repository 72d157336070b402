/*
 * tpshard_tuning.h - launch-choice variants of libtpshard's entry points, exported by the
 * separate tuning library libtpshard_tuning.so (tests and measurements only; the product
 * library libtpshard.so exports none of these and keeps no state that selects kernels).
 *
 * Each tpt_X takes the arguments of tp_X / X in tpshard.h, in the same order, followed by
 * the launch choices:
 *   tile      -1: automatic; 0..6 force the GEMM tile 256x256, 256x128, 128x128, 128x256,
 *             256x224, 128x64, 64x64 (output rows x columns per workgroup). The fp8 GEMM
 *             takes 0 or 2 and treats any other value as automatic.
 *   path      -1: automatic; 0: register-staged operands; 1: direct-to-LDS loads (needs
 *             K % 32 == 0 and no RMSNorm transform; a call that cannot use it returns
 *             TP_ERR_HIP).
 *   lm_shape  -1: the default LM-head kernel; otherwise an index into the LM head's launch
 *             shapes (tpt_lm_head_shape_count() of them).
 * An unknown choice returns TP_ERR_INVALID_ARG before any check of the other arguments.
 * Error messages are read with this library's own tp_last_error().
 */
#ifndef TPSHARD_TUNING_H
#define TPSHARD_TUNING_H

#include "tpshard.h"

#ifdef __cplusplus
extern "C" {
#endif

TP_API int tpt_column_linear(const void* x, int64_t M, int64_t K, const void* w_shard, const void* bias_shard,
                             const int64_t* subparam_sizes, int n_sub, int tp_size, int rank, int act, void* y,
                             int y_dtype, int layout, int64_t ldy, void* stream, int tile, int path);
TP_API int tpt_column_linear_fp8(const void* x_q, const float* x_scale, int64_t M, int64_t K, const void* w_q,
                                 const float* w_scale, const void* bias_shard, const int64_t* subparam_sizes,
                                 int n_sub, int tp_size, int rank, int act, void* y, int y_dtype, int layout,
                                 int64_t ldy, void* stream, int tile);
TP_API int tpt_row_linear_partial(const void* x_shard, int64_t M, int64_t K_logical, int64_t N, const void* w_shard,
                                  const void* bias, int tp_size, int rank, float* y_partial, int accumulate,
                                  void* stream, int tile, int path);
TP_API int tpt_qwi_swiglu(const void* xnorm, int64_t M, int64_t E, int64_t heads, int64_t padded_heads, int64_t qkv,
                          int64_t ff, int tp_size, int rank, const void* w_qwi, void* q, void* y_fused, void* stream,
                          int tile, int path);
TP_API int tpt_o_wo_partial(const void* y_fused, int64_t M, int64_t heads, int64_t padded_heads, int64_t qkv,
                            int64_t ff, int64_t E, int tp_size, int rank, const void* w_o, float* y_partial,
                            int accumulate, void* stream, int tile, int path);
TP_API int tpt_rmsnorm_column_linear(const void* x, int64_t M, int64_t K, const void* scale, float eps,
                                     void* xnorm_out, const void* w_shard, const void* bias_shard,
                                     const int64_t* subparam_sizes, int n_sub, int tp_size, int rank, void* y,
                                     int y_dtype, int layout, int64_t ldy, void* workspace, size_t workspace_bytes,
                                     void* stream, int tile, int path);
TP_API int tpt_lm_head_shard_argmax(const void* x, int64_t B, int64_t K, int64_t vocab, int tp_size, int rank,
                                    int64_t max_rows_per_chunk, const void* w_shard, int w_dtype,
                                    const float* w_block_scale, float* logits, int32_t* argmax_local,
                                    float* max_logit, void* workspace, size_t workspace_bytes, void* stream,
                                    int lm_shape);
/* The RMSNorm pass of rmsnorm_column_linear alone (no GEMM): the same arguments, xnorm_out
 * required, the workspace at least tp_rmsnorm_workspace_min_bytes(M, K). For measurements that
 * time the column GEMM under the conditions of the full call (the pass runs just before it). */
TP_API int tpt_rmsnorm_rows(const void* x, int64_t M, int64_t K, const void* scale, float eps, void* xnorm_out,
                            void* workspace, size_t workspace_bytes, void* stream);

/* The automatic tile for an M x N x K bf16 GEMM and for an E4M3 one (-1 for invalid sizes),
 * and the number of LM-head launch shapes. */
TP_API int tpt_gemm_pick_tile(int64_t M, int64_t N, int64_t K);
TP_API int tpt_gemm_fp8_pick_tile(int64_t M, int64_t N, int64_t K);
TP_API int tpt_lm_head_shape_count(void);

/* One matrix instruction on fixed operands, to observe its rounding: A holds 32 rows (fp8 = 0:
 * [32][16] bf16 values; fp8 = 1: [32][64] E4M3 codes), B is all ones and C[i] is added to row
 * i, so out[i] = C[i] + the sum of row i's values as the instruction computes it (one wave;
 * a: device, 16-byte aligned; c, out: device f32 [32]). TP_ERR_HIP for a failed launch. */
TP_API int tpt_mfma_row_sums(int fp8, const void* a, const float* c, float* out, void* stream);

/* Streams `rows` rows of 8192 bytes (w: device, 16-byte aligned, rows >= 64) once with 16-byte
 * loads in fetch shape `shape` (what one load instruction covers: 0 = 16 rows x 64 B, 1 = 8 rows
 * x 128 B, 2 = 4 rows x 256 B, 3 = 1 row x 1 KB with the wave's rows interleaved, 4 = 1 row x 1 KB
 * with each wave's 64 KB in order, 5 = each 64-row block in order, 6 = the row-quad LM-head
 * kernel's order: 4 rows x 256 B, window by window over the wave's half of each 512-byte slice;
 * 7 = 6 with the slices visited from slice (block mod 16) on), non-temporal if
 * `nontemporal`; one workgroup of 8 waves per 64-row block (the last block clamped to the last
 * 64 rows). out: device, 4 bytes per block, written only in the practically impossible case
 * that the loaded words reduce to a fixed value. TP_ERR_SHAPE for a shape outside 0..7 or rows
 * outside [64, 2^20]. */
TP_API int tpt_stream_probe(int shape, int nontemporal, const void* w, int64_t rows, void* out, void* stream);

/* `workgroups` workgroups of 4 waves, each wave running `iters` rounds of four independent
 * v_mfma_f32_32x32x16_bf16 (32768 flops each; fp8 = 1: v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3,
 * 131072 flops each) on pseudo-random register operands, no memory traffic. out: device, 4 bytes
 * per workgroup, practically never written. TP_ERR_SHAPE for workgroups outside [1, 2^20] or
 * iters < 1. */
TP_API int tpt_mfma_rate(int fp8, int workgroups, int iters, void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TPSHARD_TUNING_H */
