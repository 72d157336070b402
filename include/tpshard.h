/*
 * tpshard.h - C ABI of one tensor-parallel rank's share of a transformer block's
 * linear layers, native to AMD Instinct MI355X (gfx950).
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Tensors are row-major with the last dimension contiguous. "Device" pointers
 *    are HIP device memory of the current device; "host" pointers are ordinary
 *    CPU memory read before the call returns.
 *  - bf16 tensors hold bfloat16 bit patterns (uint16); fp8 tensors hold OCP
 *    E4M3FN bytes; f32 tensors hold IEEE float32.
 *  - Device tensor pointers must be 16-byte aligned and the input rows (K) must
 *    keep 16-byte alignment (K a multiple of 8 bf16 values) unless an entry point
 *    says otherwise; output leading dimensions are free.
 *  - Weights are [out_features, in_features] (the input dimension contiguous):
 *    the linear computes y = x W^T (+ b).
 *  - The caller allocates and owns every buffer, including workspaces. The
 *    library allocates no memory and never synchronises: work is enqueued on
 *    `stream` (a hipStream_t; NULL is the null stream) and the call returns.
 *  - Every argument check runs on the host before any HIP call. A failed check
 *    returns a non-zero tp_status and enqueues nothing; tp_last_error() then
 *    returns a message for the calling thread. A launch failure reported by the
 *    HIP runtime returns TP_ERR_HIP.
 *  - Ranks are arguments, not processes: one GPU computes any rank's share.
 *
 * Sources (web pages on tensor-parallel linear layers):
 *  [nanotron]  nanotron rules page "Tensor-Parallel Component Patterns",
 *              sections "Attention Module" and "MLP Module".
 *  [deepspeed] DeepSpeed module_inject/layers.py, class SubParamLinearLayer
 *              (docstring, __init__, forward).
 *  [palm]      google-research scaling_transformer_inference_efficiency
 *              layers/two_d_parallel_xmap.py: allgather_layernorm, embed_manual,
 *              unembed_manual, _transformer_layer_weight_stationary,
 *              transformer_layer_weight_gathered.
 *  [tt]        Tenstorrent models/common/modules/lm_head/lm_head_1d.py:
 *              module docstring, LMHead1DConfig, LMHead1D.forward,
 *              LMHead1D.from_model_args.
 */
#ifndef TPSHARD_H
#define TPSHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every entry point below is exported from libtpshard.so; nothing else is. */
#if defined(__GNUC__) || defined(__clang__)
#define TP_API __attribute__((visibility("default")))
#else
#define TP_API
#endif

typedef enum {
  TP_OK = 0,
  TP_ERR_INVALID_ARG = 1, /* null pointer, tp_size < 1, rank outside [0, tp_size), non-positive size */
  TP_ERR_SHAPE = 2,       /* sizes that do not fit together (sub-param < tp_size, bias length, chunking, workspace) */
  TP_ERR_UNSUPPORTED = 3, /* alignment, K not a multiple of 8 (128 for fp8), unknown dtype/act/layout code */
  TP_ERR_HIP = 4          /* the HIP runtime reported an error for a launch */
} tp_status;

typedef enum { TP_DTYPE_BF16 = 0, TP_DTYPE_F32 = 1, TP_DTYPE_FP8_E4M3 = 2 } tp_dtype;
typedef enum { TP_ACT_NONE = 0, TP_ACT_GELU_ERF = 1 } tp_act;
typedef enum { TP_LAYOUT_LOCAL = 0, TP_LAYOUT_LOGICAL = 1 } tp_layout;

/* Largest number of sub-parameters one column-parallel weight may hold. */
#define TP_MAX_SUBPARAMS 16
#define TP_MAX_RANKS 64 /* most ranks tp_reduce_scatter_residual sums */

/*
 * tp_shard_widths - the rows of each sub-parameter that rank `rank` owns.
 *
 * [deepspeed] SubParamLinearLayer: a weight whose output dimension holds several
 * logical sub-parameters (fused q/k/v with unequal GQA widths, chunked MLP) is
 * partitioned sub-parameter by sub-parameter, and the per-rank widths are
 * resolved once per model. [nanotron]: local sizes are `n // tp_size`.
 * Where tp_size does not divide a size, the split is balanced and the
 * remainder goes to the lowest ranks: w_s(r) = S_s / tp + (r < S_s % tp).
 *
 * subparam_sizes  host, n_sub logical sizes S_0..S_{n-1} (each >= tp_size)
 * width           host out, n_sub: rows of each sub-parameter owned by `rank`
 * logical_off     host out, n_sub: first logical row owned in each sub-parameter
 * local_off       host out, n_sub: first row of each piece inside the rank's shard
 * shard_total     host out, 1: rows of the rank's materialised shard
 * The shard is the concatenation, in sub-parameter order, of the logical rows
 * [logical_off[s], logical_off[s] + width[s]). Pure host arithmetic; any output
 * pointer may be NULL. Errors: TP_ERR_INVALID_ARG, TP_ERR_SHAPE.
 */
TP_API int tp_shard_widths(const int64_t* subparam_sizes, int n_sub, int tp_size, int rank,
                    int64_t* width, int64_t* logical_off, int64_t* local_off, int64_t* shard_total);

/*
 * tp_column_linear - one rank's column-parallel linear with sub-parameter sharding.
 *
 * [deepspeed] SubParamLinearLayer.forward: the replicated input times the
 * transposed shard weight, plus the shard bias. [nanotron] MLP: c_fc keeps
 * intermediate // tp output columns per rank, then F.gelu.
 *
 * x           device bf16 [M, K]
 * w_shard     device bf16 [N_r, K], N_r = shard total of (subparam_sizes, tp_size, rank):
 *             the rank's rows of every sub-parameter, concatenated in sub-parameter order
 * bias_shard  device bf16 [N_r] (the same row map) or NULL
 * act         TP_ACT_NONE or TP_ACT_GELU_ERF (exact erf GELU of the float32 accumulator)
 * y           device, y_dtype TP_DTYPE_BF16 or TP_DTYPE_F32:
 *             TP_LAYOUT_LOCAL:   [M, ldy], ldy >= N_r; local column j is written at j
 *             TP_LAYOUT_LOGICAL: [M, ldy], ldy >= sum(subparam_sizes); local column j of
 *             sub-parameter s is written at its logical column
 *             logical_off[s] + (j - local_off[s]); other columns are not touched
 * Each output is rounded once: y = round(act(f32 sum_k x w + b)).
 * M = 0 is an empty input: nothing is enqueued and x, y may be NULL.
 * Errors: TP_ERR_INVALID_ARG, TP_ERR_SHAPE, TP_ERR_UNSUPPORTED (K % 8, misalignment),
 * TP_ERR_HIP.
 */
TP_API int tp_column_linear(const void* x, int64_t M, int64_t K, const void* w_shard, const void* bias_shard,
                     const int64_t* subparam_sizes, int n_sub, int tp_size, int rank, int act, void* y,
                     int y_dtype, int layout, int64_t ldy, void* stream);

/*
 * tp_quantize_rows_e4m3 - per-row (per-token) E4M3 quantisation of bf16 activations, the
 * first step of the fp8 prefill linear below.
 *
 * [palm] transformer_layer_weight_gathered: a QuantizedLayer multiplies by quantised
 * weights and applies the per-output-channel scale to the matmul result. To run that
 * product on fp8 matrix cores the activations are quantised too, one scale per row:
 * scale[m] = amax_k |x[m,k]| / 448 (1 for an all-zero row), q[m,k] = e4m3(x[m,k] / scale[m]),
 * both divisions IEEE float32 (nearest even), the code the nearest E4M3 value (ties to the
 * even mantissa, 448 and beyond saturate to 448, sign from the float's sign bit).
 *
 * x      device bf16 [M, K], 16-byte aligned; K % 8 == 0
 * q      device uint8 [M, K] (OCP E4M3FN codes), 16-byte aligned
 * scale  device f32 [M]
 * M = 0 enqueues nothing. Errors: TP_ERR_INVALID_ARG, TP_ERR_UNSUPPORTED (K % 8,
 * misalignment), TP_ERR_HIP.
 */
TP_API int tp_quantize_rows_e4m3(const void* x, int64_t M, int64_t K, void* q, float* scale, void* stream);

/*
 * tp_column_linear_fp8 - tp_column_linear on E4M3 activations and weights (fp8 prefill).
 *
 * [palm] QuantizedLayer: y = round(act(x_scale[m] * w_scale[j] * sum_k q_x[m,k] q_w[j,k]
 * + b[j])), the product of E4M3 values accumulated in float32 on the fp8 matrix cores, the
 * per-output-channel weight scale (and the per-row activation scale) applied to the product.
 *
 * x_q       device uint8 [M, K]: E4M3 codes (tp_quantize_rows_e4m3), x_scale device f32 [M]
 * w_q       device uint8 [N_r, K]: E4M3 codes of the rank's weight rows, w_scale f32 [N_r]
 *           (one scale per output channel), same row map as tp_column_linear
 * K % 64 == 0. Everything else (bias, act, y, y_dtype, layout, ldy, M = 0) as
 * tp_column_linear. Errors: as tp_column_linear, TP_ERR_UNSUPPORTED for K % 64 and for
 * operands whose rows within one tile (up to 256 of them) span more than 2^31 - 1 bytes.
 */
TP_API int tp_column_linear_fp8(const void* x_q, const float* x_scale, int64_t M, int64_t K, const void* w_q,
                                const float* w_scale, const void* bias_shard, const int64_t* subparam_sizes,
                                int n_sub, int tp_size, int rank, int act, void* y, int y_dtype, int layout,
                                int64_t ldy, void* stream);

/*
 * tp_vocab_embedding - one rank's share of the vocab-parallel embedding lookup.
 *
 * [palm] embed_manual: each device holds the embedding rows of its vocab shard; a token id
 * minus the shard's first id indexes the table, and tokens outside the shard give a zero
 * row, so the ranks' outputs sum (the page's reduce-scatter) to the full lookup.
 *
 * tokens       device int32 [n_tokens]; ids outside [0, vocab) give a zero row on every rank
 * vocab, tp_size, rank  the shard is tp_shard_widths({vocab}, ...): rows [off, off + V_r)
 * table_shard  device bf16 [V_r, E], 16-byte aligned; E % 8 == 0
 * out          device bf16 [n_tokens, E], 16-byte aligned
 * n_tokens = 0 enqueues nothing. Errors: TP_ERR_INVALID_ARG, TP_ERR_SHAPE (vocab < tp_size),
 * TP_ERR_UNSUPPORTED (E % 8, misalignment, sizes beyond 31 bits), TP_ERR_HIP.
 */
TP_API int tp_vocab_embedding(const int32_t* tokens, int64_t n_tokens, int64_t vocab, int tp_size, int rank,
                              const void* table_shard, int64_t E, void* out, void* stream);

/*
 * tp_qwi_swiglu - one rank's fused q_wi projection with the SwiGLU of its MLP columns.
 *
 * [palm] q_wi and SwiGLU steps of the transformer layers: one product of the normalised
 * input with each head's q_wi weight gives the head's qkv query columns, then wi0 and wi1
 * of fph = ff / (heads - padded_heads) columns each (integer division: the d_ff width is
 * spread over the real heads); the MLP activation is swish(wi0) * wi1 at the full d_ff
 * width. Heads split evenly over ranks: the rank holds h_r = heads / tp_size of them.
 * Per output: wi0 and wi1 are float32 accumulators rounded to bf16, then
 * y = bf16(wi0 / (1 + exp(-wi0)) * wi1) (Swish with unit slope) in float32.
 *
 * xnorm     device bf16 [M, E], E % 8 == 0
 * heads     all heads, padding included (heads % tp_size == 0); 0 <= padded_heads < heads
 * w_qwi     device bf16 [h_r * (qkv + 2 fph), E]: the rank's heads in order, each head's
 *           qkv query rows, then its fph wi0 rows, then its fph wi1 rows (the page's
 *           [heads, E, q_wi_per_head] shard with the output axis first, E contiguous)
 * q         device bf16 [M, h_r, qkv], or NULL to skip the query columns
 * y_fused   device bf16 [M, h_r, qkv + fph]: y is written at [m, h, qkv + j]; the
 *           attention slots [m, h, 0:qkv] are left as they are (the page concatenates the
 *           attention output there before the o_wo projection)
 * All pointers 16-byte aligned. M = 0 enqueues nothing. Errors: TP_ERR_INVALID_ARG,
 * TP_ERR_SHAPE (heads % tp_size, fph < 1), TP_ERR_UNSUPPORTED (E % 8, misalignment,
 * sizes beyond 31 bits), TP_ERR_HIP.
 */
TP_API int tp_qwi_swiglu(const void* xnorm, int64_t M, int64_t E, int64_t heads, int64_t padded_heads, int64_t qkv,
                         int64_t ff, int tp_size, int rank, const void* w_qwi, void* q, void* y_fused, void* stream);

/*
 * tp_o_wo_partial - one rank's fused attention-out and MLP-out projection, before any
 * reduction.
 *
 * [palm] o_wo step: y_out[m, e] = sum over the rank's heads h and each head's qkv + fph
 * positions d of y_fused[m, h, d] * o_wo[h, d, e], a float32 partial that the page then
 * reduce-scatters over the devices holding the other heads. Dimensions as tp_qwi_swiglu.
 *
 * y_fused    device bf16 [M, h_r, qkv + fph]; h_r (qkv + fph) % 8 == 0
 * w_o        device bf16 [E, h_r (qkv + fph)] (the page's [heads, d, E] shard transposed,
 *            the contraction axis contiguous)
 * y_partial  device f32 [M, E]; accumulate = 1 adds to the values there (one rounding)
 * Errors: as tp_qwi_swiglu; TP_ERR_UNSUPPORTED when h_r (qkv + fph) % 8 != 0.
 */
TP_API int tp_o_wo_partial(const void* y_fused, int64_t M, int64_t heads, int64_t padded_heads, int64_t qkv,
                           int64_t ff, int64_t E, int tp_size, int rank, const void* w_o, float* y_partial,
                           int accumulate, void* stream);

/*
 * tp_reduce_scatter_residual - one rank's output of the sequence-parallel reduce-scatter of
 * the ranks' row-parallel partials, with the residual add (all ranks' partials on one GPU).
 *
 * [nanotron] MLP Module: c_proj, a row-parallel linear, returns [batch, seq / tp, hidden] on
 * each rank; [palm] reduce-scatters the o_wo partials, then adds the residual,
 * z = bf16(y_out + x). Rank dest_rank keeps positions [dest_rank sl, (dest_rank + 1) sl) of
 * every sequence, sl = seq / tp_size. Output row i = b sl + t sums, in rank order and in
 * float32, row b seq + dest_rank sl + t of every partial: S = ((P_0 + P_1) + ...) + P_tp-1.
 *
 * partials   host array of tp_size device pointers, rank r's f32 partial [batch seq, N]
 *            (tp_row_linear_partial, tp_o_wo_partial); read before the call returns
 * tp_size    1..TP_MAX_RANKS; seq % tp_size == 0; N % 4 == 0
 * residual   device bf16 [batch sl, N] (the rank's slice of the residual stream) or NULL
 * z          device bf16 [batch sl, N]: bf16(S + residual) (bf16(S) without one), or NULL
 * y_sum      device f32 [batch sl, N]: S, or NULL; z and y_sum are not both NULL when batch > 0
 * All device pointers 16-byte aligned. batch = 0 enqueues nothing. Errors:
 * TP_ERR_INVALID_ARG, TP_ERR_SHAPE (seq % tp_size), TP_ERR_UNSUPPORTED (N % 4, misalignment),
 * TP_ERR_HIP.
 */
TP_API int tp_reduce_scatter_residual(const float* const* partials, int tp_size, int64_t batch, int64_t seq,
                                      int64_t N, int dest_rank, const void* residual, void* z, float* y_sum,
                                      void* stream);

/*
 * tp_row_linear_partial - one rank's row-parallel partial sum, before any reduction.
 *
 * [nanotron] TensorParallelRowLinear (the MLP's c_proj, the attention's output
 * projection): each rank holds a slice of the input features and the matching
 * weight columns; its product is the rank's float32 partial of the full output,
 * which the pages then reduce across ranks with a collective.
 *
 * x_shard    device bf16 [M, K_r], K_r = the rank's width of K_logical (tp_shard_widths)
 * w_shard    device bf16 [N, K_r]
 * bias       device bf16 [N] or NULL; added by rank 0 only, so the ranks' partials sum
 *            to the unsharded output
 * y_partial  device f32 [M, N]; accumulate = 0 stores the partial, accumulate = 1 adds it
 *            to the values already there with one float32 rounding (a rank-ordered sum
 *            when the ranks run in order)
 * Errors: as tp_column_linear; the rank's input width K_r must be a multiple of 8.
 */
TP_API int tp_row_linear_partial(const void* x_shard, int64_t M, int64_t K_logical, int64_t N, const void* w_shard,
                          const void* bias, int tp_size, int rank, float* y_partial, int accumulate,
                          void* stream);

/*
 * tp_rmsnorm_workspace_bytes     device workspace for rmsnorm_column_linear's fast path: the
 *                                row statistics plus the bf16 normalised rows [M, K], which the
 *                                GEMM then reads with direct-to-LDS loads.
 * tp_rmsnorm_workspace_min_bytes the least workspace it accepts (row statistics only): the
 *                                normalisation is then fused into the GEMM's A staging.
 */
TP_API size_t tp_rmsnorm_workspace_bytes(int64_t M, int64_t K);
TP_API size_t tp_rmsnorm_workspace_min_bytes(int64_t M, int64_t K);

/*
 * rmsnorm_column_linear - RMSNorm of each input row, then the rank's column linear on it.
 *
 * [palm] allgather_layernorm: float32 statistics, r = rsqrt(mean(x^2) + eps),
 * n = bf16(x * r); with a learned scale the page first adds 1 to the bf16 scale
 * (the T5X option that centres the learned scale at zero), so t = bf16(1 + s) and y = bf16(n * t).
 * transformer_layer_weight_gathered normalises without a scale (scale = NULL).
 * One device holds whole rows, so the page's mean across shards is the mean of
 * the row. The library sums the exact squares in float64 and rounds r to float32
 * once (at least the page's float32 precision; no finite row overflows).
 *
 * x          device bf16 [M, K]
 * scale      device bf16 [K] or NULL
 * eps        added to the mean square (the pages use 1e-6)
 * xnorm_out  device bf16 [M, K] receiving y, or NULL
 * w_shard, bias_shard, subparam_sizes, n_sub, tp_size, rank, y, y_dtype, layout, ldy:
 *            as tp_column_linear, with y's input rows being the normalised rows
 * workspace  device, 256-byte aligned, contents need no initialisation (scratch between
 *            calls). With xnorm_out, or with tp_rmsnorm_workspace_bytes(M, K) bytes, the
 *            normalised rows are materialised and multiplied; with at least
 *            tp_rmsnorm_workspace_min_bytes(M, K) bytes the normalisation is fused into the
 *            GEMM's A staging. Both give bit-identical y.
 * Errors: as tp_column_linear, TP_ERR_SHAPE for a short workspace.
 */
TP_API int rmsnorm_column_linear(const void* x, int64_t M, int64_t K, const void* scale, float eps, void* xnorm_out,
                          const void* w_shard, const void* bias_shard, const int64_t* subparam_sizes, int n_sub,
                          int tp_size, int rank, void* y, int y_dtype, int layout, int64_t ldy, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * tp_lm_head_workspace_bytes - device workspace lm_head_shard_argmax needs: enough for any
 * batch size, any max_rows_per_chunk and any of the library's launch shapes (256 bytes per
 * row of the rank's vocab shard). B, vocab, tp_size and rank are checked as in
 * lm_head_shard_argmax; 0 for invalid arguments.
 */
TP_API size_t tp_lm_head_workspace_bytes(int64_t B, int64_t vocab, int tp_size, int rank);

/*
 * lm_head_shard_argmax - a vocab shard's float32 logits and per-row argmax (decode).
 *
 * [tt] LMHead1D: the output projection of each device's vocab shard is split
 * into chunks of at most max_rows_per_chunk rows (every chunk but the last has
 * that many rows, the last the remainder), one linear runs per chunk and the
 * outputs are concatenated, so each device holds the complete logits of its own
 * vocab rows (column-parallel, no partial sums); the argmax across devices is
 * left to the caller. [palm] unembed_manual computes logits in float32.
 *
 * x                 device bf16 [B, K]
 * vocab, tp_size, rank  the shard is tp_shard_widths({vocab}, ...): V_r rows starting
 *                   at vocab id logical_off (returned indices are local to the shard)
 * w_shard           device [V_r, K], w_dtype TP_DTYPE_BF16 or TP_DTYPE_FP8_E4M3
 * w_block_scale     fp8 only: device f32 [V_r, K / 128], the scale of each row's
 *                   128-wide K block (value = scale * E4M3 value); NULL for bf16
 * logits            device f32 [B, V_r]; chunk c's rows land at columns c*max_rows_per_chunk...
 * argmax_local      device int32 [B]: lowest local index of the row's largest logit
 * max_logit         device f32 [B] or NULL: that largest logit
 * workspace         device, tp_lm_head_workspace_bytes(...) bytes, 256-byte aligned; needs
 *                   no initialisation (per-workgroup argmax candidates, scratch between
 *                   calls). Calls that overlap in time must not share a workspace.
 * Two kernels run per pass over the weight: the logits with per-workgroup argmax candidates,
 * then the candidates' reduction. A pass takes up to 32 batch rows, or up to 64 when the call
 * has more than 32 (then x stays in LDS and the weight streams once per 64 rows).
 * Errors: TP_ERR_INVALID_ARG, TP_ERR_SHAPE (chunk size <= 0, workspace short),
 * TP_ERR_UNSUPPORTED (K % 8, fp8 with K % 128, dtype), TP_ERR_HIP.
 */
TP_API int lm_head_shard_argmax(const void* x, int64_t B, int64_t K, int64_t vocab, int tp_size, int rank,
                         int64_t max_rows_per_chunk, const void* w_shard, int w_dtype, const float* w_block_scale,
                         float* logits, int32_t* argmax_local, float* max_logit, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * lm_head_shard_argmax_noalloc - lm_head_shard_argmax for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments without the workspace, the same results bit for bit.
 *
 * The per-workgroup candidates go to a device array of 1 MiB inside the library, one copy per
 * GPU, which the library holds until the process ends (its address is looked up on the first
 * call on each device). The call allocates nothing. Shards whose candidates do not fit (more
 * than 262144 vocab rows, or 131072 when more than 32 batch rows share a weight pass) return
 * TP_ERR_SHAPE before anything is enqueued. Every call on one GPU shares that GPU's array: calls
 * that overlap in time on one GPU (other streams, other threads) race and must be ordered by
 * the caller. Nothing in the array needs initialisation. Errors: as lm_head_shard_argmax, and
 * TP_ERR_HIP when the array's address cannot be found.
 */
TP_API int lm_head_shard_argmax_noalloc(const void* x, int64_t B, int64_t K, int64_t vocab, int tp_size, int rank,
                                        int64_t max_rows_per_chunk, const void* w_shard, int w_dtype,
                                        const float* w_block_scale, float* logits, int32_t* argmax_local,
                                        float* max_logit, void* stream);

/*
 * tp_last_error - message of the last non-OK status returned on the calling thread
 * ("" if none). The pointer stays valid until the thread's next call into the library.
 */
TP_API const char* tp_last_error(void);

/*
 * tp_version - library version string (static storage).
 */
TP_API const char* tp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TPSHARD_H */
