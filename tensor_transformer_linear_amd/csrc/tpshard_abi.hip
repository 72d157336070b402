// C ABI of libtpshard: argument checks, shard arithmetic and kernel dispatch.
//
// Every check runs on the host before any HIP call; a failed check sets the
// calling thread's message and returns a status without touching the GPU. The
// exported calls hold no state of their own: each passes the automatic launch
// choices to its internal body (abi_impl.h).
#include <limits.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "abi_impl.h"
#include "common.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return TP_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// The balanced split with the remainder on the lowest ranks.
int64_t width_of(int64_t size, int tp, int r) { return size / tp + (r < size % tp ? 1 : 0); }

struct Shard {
  int n_sub;
  int64_t width[TP_MAX_SUBPARAMS], logical_off[TP_MAX_SUBPARAMS], local_off[TP_MAX_SUBPARAMS];
  int64_t total, logical_total;
};

int resolve_shard(const int64_t* sizes, int n_sub, int tp_size, int rank, Shard* s) {
  if (sizes == nullptr) return fail(TP_ERR_INVALID_ARG, "subparam_sizes is NULL");
  if (n_sub < 1 || n_sub > TP_MAX_SUBPARAMS)
    return fail(TP_ERR_INVALID_ARG, "n_sub = %d outside [1, %d]", n_sub, TP_MAX_SUBPARAMS);
  if (tp_size < 1) return fail(TP_ERR_INVALID_ARG, "tp_size = %d must be >= 1", tp_size);
  if (rank < 0 || rank >= tp_size) return fail(TP_ERR_INVALID_ARG, "rank %d outside [0, %d)", rank, tp_size);
  s->n_sub = n_sub;
  int64_t base = 0, local = 0;
  for (int i = 0; i < n_sub; ++i) {
    const int64_t S = sizes[i];
    if (S <= 0) return fail(TP_ERR_INVALID_ARG, "sub-parameter %d has size %lld", i, (long long)S);
    if (S < tp_size)
      return fail(TP_ERR_SHAPE, "sub-parameter %d has size %lld, smaller than tp_size %d", i, (long long)S, tp_size);
    if (S > (int64_t)INT_MAX || base > (int64_t)INT_MAX - S)
      return fail(TP_ERR_UNSUPPORTED, "logical output width exceeds %d", INT_MAX);
    int64_t before = 0;
    for (int q = 0; q < rank; ++q) before += width_of(S, tp_size, q);
    s->width[i] = width_of(S, tp_size, rank);
    s->logical_off[i] = base + before;
    s->local_off[i] = local;
    local += s->width[i];
    base += S;
  }
  s->total = local;
  s->logical_total = base;
  return TP_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(TP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Checks shared by the column-parallel entry points; fills the GEMM problem.
int prepare_column(const void* x, int64_t M, int64_t K, const void* w_shard, const void* bias_shard,
                   const int64_t* subparam_sizes, int n_sub, int tp_size, int rank, int act, void* y, int y_dtype,
                   int layout, int64_t ldy, tpk::GemmProblem* p) {
  Shard sh;
  int st = resolve_shard(subparam_sizes, n_sub, tp_size, rank, &sh);
  if (st != TP_OK) return st;
  if (M < 0) return fail(TP_ERR_INVALID_ARG, "M = %lld must be >= 0", (long long)M);
  if (w_shard == nullptr) return fail(TP_ERR_INVALID_ARG, "w_shard must be non-NULL");
  if (M > 0 && (x == nullptr || y == nullptr)) return fail(TP_ERR_INVALID_ARG, "x and y must be non-NULL");
  if (K <= 0) return fail(TP_ERR_INVALID_ARG, "K = %lld must be positive", (long long)K);
  if (M > INT_MAX || K > INT_MAX) return fail(TP_ERR_UNSUPPORTED, "M and K must fit in 31 bits");
  if (K % 8) return fail(TP_ERR_UNSUPPORTED, "K = %lld must be a multiple of 8", (long long)K);
  if (act != TP_ACT_NONE && act != TP_ACT_GELU_ERF) return fail(TP_ERR_UNSUPPORTED, "unknown act %d", act);
  if (y_dtype != TP_DTYPE_BF16 && y_dtype != TP_DTYPE_F32)
    return fail(TP_ERR_UNSUPPORTED, "y_dtype %d: output must be bf16 or f32", y_dtype);
  if (layout != TP_LAYOUT_LOCAL && layout != TP_LAYOUT_LOGICAL) return fail(TP_ERR_UNSUPPORTED, "unknown layout %d", layout);
  const int64_t need = layout == TP_LAYOUT_LOCAL ? sh.total : sh.logical_total;
  if (ldy < need)
    return fail(TP_ERR_SHAPE, "ldy = %lld is smaller than the %s output width %lld", (long long)ldy,
                layout == TP_LAYOUT_LOCAL ? "local" : "logical", (long long)need);
  if (!aligned(x, 16) || !aligned(w_shard, 16) || !aligned(y, 16))
    return fail(TP_ERR_UNSUPPORTED, "x, w_shard and y must be 16-byte aligned");
  if (bias_shard != nullptr && !aligned(bias_shard, 2)) return fail(TP_ERR_UNSUPPORTED, "bias_shard misaligned");

  memset(p, 0, sizeof(*p));
  p->A = static_cast<const uint16_t*>(x);
  p->lda = K;
  p->B = static_cast<const uint16_t*>(w_shard);
  p->ldb = K;
  p->M = (int)M;
  p->N = (int)sh.total;
  p->K = (int)K;
  p->ep.bias = static_cast<const uint16_t*>(bias_shard);
  p->ep.C = y;
  p->ep.ldc = ldy;
  p->ep.act = act;
  p->ep.out_f32 = y_dtype == TP_DTYPE_F32;
  p->ep.accumulate = 0;
  p->ep.n_seg = 0;
  if (layout == TP_LAYOUT_LOGICAL) {
    p->ep.n_seg = sh.n_sub;
    for (int i = 0; i < sh.n_sub; ++i) {
      p->ep.seg_end[i] = (int)(sh.local_off[i] + sh.width[i]);
      p->ep.seg_delta[i] = (int)(sh.logical_off[i] - sh.local_off[i]);
    }
  }
  return TP_OK;
}

// Head dimensions of the fused q_wi / o_wo layers: heads split evenly over ranks, the MLP
// width spread over the real heads.
struct HeadDims {
  int64_t h_r, fph, qph, fused;  // heads per rank, MLP columns per head, q_wi rows per head, y_fused columns per head
};

int resolve_heads(int64_t heads, int64_t padded_heads, int64_t qkv, int64_t ff, int tp_size, int rank, HeadDims* d) {
  if (tp_size < 1) return fail(TP_ERR_INVALID_ARG, "tp_size = %d must be >= 1", tp_size);
  if (rank < 0 || rank >= tp_size) return fail(TP_ERR_INVALID_ARG, "rank %d outside [0, %d)", rank, tp_size);
  if (heads < 1 || qkv < 1 || ff < 1)
    return fail(TP_ERR_INVALID_ARG, "heads = %lld, qkv = %lld, ff = %lld must be positive", (long long)heads,
                (long long)qkv, (long long)ff);
  if (padded_heads < 0 || padded_heads >= heads)
    return fail(TP_ERR_INVALID_ARG, "padded_heads = %lld outside [0, heads = %lld)", (long long)padded_heads,
                (long long)heads);
  if (heads % tp_size)
    return fail(TP_ERR_SHAPE, "heads = %lld do not split evenly over tp_size %d", (long long)heads, tp_size);
  if (heads > INT_MAX || qkv > INT_MAX || ff > INT_MAX) return fail(TP_ERR_UNSUPPORTED, "sizes must fit in 31 bits");
  d->h_r = heads / tp_size;
  d->fph = ff / (heads - padded_heads);
  if (d->fph < 1)
    return fail(TP_ERR_SHAPE, "ff = %lld is smaller than the %lld real heads", (long long)ff,
                (long long)(heads - padded_heads));
  d->qph = qkv + 2 * d->fph;
  d->fused = qkv + d->fph;
  if (d->h_r * d->qph > INT_MAX / 2) return fail(TP_ERR_UNSUPPORTED, "the rank's q_wi rows must fit in 30 bits");
  return TP_OK;
}

}  // namespace

namespace tpabi {

int check_tuning(const Tuning& t) {
  if (t.tile < tpk::TILE_AUTO || t.tile >= tpk::TILE_COUNT) return fail(TP_ERR_INVALID_ARG, "unknown tile %d", t.tile);
  if (t.path < tpk::GEMM_PATH_AUTO || t.path > tpk::GEMM_PATH_DMA)
    return fail(TP_ERR_INVALID_ARG, "unknown path %d", t.path);
  if (t.lm_shape < -1 || t.lm_shape >= tpk::lm_head_shape_count())
    return fail(TP_ERR_INVALID_ARG, "unknown LM-head shape %d", t.lm_shape);
  return TP_OK;
}

int column_linear(const void* x, int64_t M, int64_t K, const void* w_shard, const void* bias_shard,
                  const int64_t* subparam_sizes, int n_sub, int tp_size, int rank, int act, void* y, int y_dtype,
                  int layout, int64_t ldy, void* stream, const Tuning& tune) {
  tpk::GemmProblem p;
  int st = prepare_column(x, M, K, w_shard, bias_shard, subparam_sizes, n_sub, tp_size, rank, act, y, y_dtype, layout,
                          ldy, &p);
  if (st != TP_OK) return st;
  if (M == 0) return ok();
  return hip_status(tpk::launch_gemm(p, tune.tile, tune.path, as_stream(stream)), "tp_column_linear launch");
}

int column_linear_fp8(const void* x_q, const float* x_scale, int64_t M, int64_t K, const void* w_q,
                      const float* w_scale, const void* bias_shard, const int64_t* subparam_sizes, int n_sub,
                      int tp_size, int rank, int act, void* y, int y_dtype, int layout, int64_t ldy, void* stream,
                      const Tuning& tune) {
  tpk::GemmProblem p;
  int st = prepare_column(x_q, M, K, w_q, bias_shard, subparam_sizes, n_sub, tp_size, rank, act, y, y_dtype, layout,
                          ldy, &p);
  if (st != TP_OK) return st;
  if (K % 64) return fail(TP_ERR_UNSUPPORTED, "K = %lld must be a multiple of 64 for the fp8 path", (long long)K);
  if (w_scale == nullptr || (M > 0 && x_scale == nullptr))
    return fail(TP_ERR_INVALID_ARG, "x_scale and w_scale must be non-NULL");
  if (!aligned(x_scale, 4) || !aligned(w_scale, 4)) return fail(TP_ERR_UNSUPPORTED, "scales must be 4-byte aligned");
  if (M == 0) return ok();
  p.fp8 = 1;
  p.ep.row_scale = x_scale;
  p.ep.col_scale = w_scale;
  const int tile = tune.tile == tpk::TILE_256x256 || tune.tile == tpk::TILE_128x128 ? tune.tile : tpk::TILE_AUTO;
  const hipError_t e = tpk::launch_gemm_fp8(p, tile, as_stream(stream));
  if (e == hipErrorNotSupported)
    return fail(TP_ERR_UNSUPPORTED, "a tile's operand rows span more than 2^31 - 1 bytes (K = %lld)", (long long)K);
  return hip_status(e, "tp_column_linear_fp8 launch");
}

int row_linear_partial(const void* x_shard, int64_t M, int64_t K_logical, int64_t N, const void* w_shard,
                       const void* bias, int tp_size, int rank, float* y_partial, int accumulate, void* stream,
                       const Tuning& tune) {
  if (tp_size < 1) return fail(TP_ERR_INVALID_ARG, "tp_size = %d must be >= 1", tp_size);
  if (rank < 0 || rank >= tp_size) return fail(TP_ERR_INVALID_ARG, "rank %d outside [0, %d)", rank, tp_size);
  if (w_shard == nullptr || (M > 0 && (x_shard == nullptr || y_partial == nullptr)))
    return fail(TP_ERR_INVALID_ARG, "x_shard, w_shard and y_partial must be non-NULL");
  if (M < 0 || N <= 0 || K_logical <= 0)
    return fail(TP_ERR_INVALID_ARG, "M = %lld, N = %lld, K_logical = %lld: need M >= 0, N > 0, K_logical > 0",
                (long long)M, (long long)N, (long long)K_logical);
  if (K_logical < tp_size)
    return fail(TP_ERR_SHAPE, "K_logical = %lld is smaller than tp_size %d", (long long)K_logical, tp_size);
  if (M > INT_MAX || N > INT_MAX || K_logical > INT_MAX) return fail(TP_ERR_UNSUPPORTED, "sizes must fit in 31 bits");
  if (accumulate != 0 && accumulate != 1) return fail(TP_ERR_INVALID_ARG, "accumulate must be 0 or 1");
  const int64_t K_r = width_of(K_logical, tp_size, rank);
  if (K_r % 8) return fail(TP_ERR_UNSUPPORTED, "the rank's input width %lld must be a multiple of 8", (long long)K_r);
  if (!aligned(x_shard, 16) || !aligned(w_shard, 16) || !aligned(y_partial, 16))
    return fail(TP_ERR_UNSUPPORTED, "x_shard, w_shard and y_partial must be 16-byte aligned");
  if (bias != nullptr && !aligned(bias, 2)) return fail(TP_ERR_UNSUPPORTED, "bias misaligned");
  if (M == 0) return ok();

  tpk::GemmProblem p;
  memset(&p, 0, sizeof(p));
  p.A = static_cast<const uint16_t*>(x_shard);
  p.lda = K_r;
  p.B = static_cast<const uint16_t*>(w_shard);
  p.ldb = K_r;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K_r;
  p.ep.bias = rank == 0 ? static_cast<const uint16_t*>(bias) : nullptr;
  p.ep.C = y_partial;
  p.ep.ldc = N;
  p.ep.act = TP_ACT_NONE;
  p.ep.out_f32 = 1;
  p.ep.accumulate = accumulate;
  return hip_status(tpk::launch_gemm(p, tune.tile, tune.path, as_stream(stream)), "tp_row_linear_partial launch");
}

int qwi_swiglu(const void* xnorm, int64_t M, int64_t E, int64_t heads, int64_t padded_heads, int64_t qkv, int64_t ff,
               int tp_size, int rank, const void* w_qwi, void* q, void* y_fused, void* stream, const Tuning& tune) {
  HeadDims d;
  int st = resolve_heads(heads, padded_heads, qkv, ff, tp_size, rank, &d);
  if (st != TP_OK) return st;
  if (M < 0 || E < 1) return fail(TP_ERR_INVALID_ARG, "M = %lld, E = %lld: need M >= 0, E > 0", (long long)M, (long long)E);
  if (w_qwi == nullptr || (M > 0 && (xnorm == nullptr || y_fused == nullptr)))
    return fail(TP_ERR_INVALID_ARG, "xnorm, w_qwi and y_fused must be non-NULL");
  if (M > INT_MAX || E > INT_MAX) return fail(TP_ERR_UNSUPPORTED, "M and E must fit in 31 bits");
  if (E % 8) return fail(TP_ERR_UNSUPPORTED, "E = %lld must be a multiple of 8", (long long)E);
  if (!aligned(xnorm, 16) || !aligned(w_qwi, 16) || !aligned(y_fused, 16) || !aligned(q, 16))
    return fail(TP_ERR_UNSUPPORTED, "xnorm, w_qwi, q and y_fused must be 16-byte aligned");
  if (M == 0) return ok();

  tpk::GemmProblem p;
  memset(&p, 0, sizeof(p));
  p.A = static_cast<const uint16_t*>(xnorm);
  p.lda = E;
  p.B = static_cast<const uint16_t*>(w_qwi);
  p.ldb = E;
  p.M = (int)M;
  p.K = (int)E;
  hipStream_t s = as_stream(stream);
  // MLP columns: output column c = h * fph + j pairs wi0 row h * qph + qkv + j with the wi1
  // row fph further and lands at y_fused[m, h, qkv + j].
  tpk::GemmProblem g = p;
  g.N = (int)(d.h_r * d.fph);
  g.b_head_w = (int)d.fph;
  g.b_head_pitch = (int)d.qph;
  g.b_head_off = (int)qkv;
  g.ep.C = y_fused;
  g.ep.ldc = d.h_r * d.fused;
  g.ep.glu = 1;
  g.ep.glu_off = (int)d.fph;
  g.ep.c_head_w = (int)d.fph;
  g.ep.c_head_pitch = (int)d.fused;
  g.ep.c_head_off = (int)qkv;
  hipError_t e = tpk::launch_gemm(g, tune.tile, tune.path, s);
  if (e != hipSuccess || q == nullptr) return hip_status(e, "tp_qwi_swiglu SwiGLU launch");
  // Query columns: output column c = h * qkv + t reads row h * qph + t, stored densely.
  tpk::GemmProblem a = p;
  a.N = (int)(d.h_r * qkv);
  a.b_head_w = (int)qkv;
  a.b_head_pitch = (int)d.qph;
  a.b_head_off = 0;
  a.ep.C = q;
  a.ep.ldc = d.h_r * qkv;
  return hip_status(tpk::launch_gemm(a, tune.tile, tune.path, s), "tp_qwi_swiglu query launch");
}

int o_wo_partial(const void* y_fused, int64_t M, int64_t heads, int64_t padded_heads, int64_t qkv, int64_t ff,
                 int64_t E, int tp_size, int rank, const void* w_o, float* y_partial, int accumulate, void* stream,
                 const Tuning& tune) {
  HeadDims d;
  int st = resolve_heads(heads, padded_heads, qkv, ff, tp_size, rank, &d);
  if (st != TP_OK) return st;
  if (M < 0 || E < 1) return fail(TP_ERR_INVALID_ARG, "M = %lld, E = %lld: need M >= 0, E > 0", (long long)M, (long long)E);
  if (w_o == nullptr || (M > 0 && (y_fused == nullptr || y_partial == nullptr)))
    return fail(TP_ERR_INVALID_ARG, "y_fused, w_o and y_partial must be non-NULL");
  if (accumulate != 0 && accumulate != 1) return fail(TP_ERR_INVALID_ARG, "accumulate must be 0 or 1");
  if (M > INT_MAX || E > INT_MAX) return fail(TP_ERR_UNSUPPORTED, "M and E must fit in 31 bits");
  const int64_t K = d.h_r * d.fused;
  if (K % 8)
    return fail(TP_ERR_UNSUPPORTED, "the rank's y_fused width %lld must be a multiple of 8", (long long)K);
  if (!aligned(y_fused, 16) || !aligned(w_o, 16) || !aligned(y_partial, 16))
    return fail(TP_ERR_UNSUPPORTED, "y_fused, w_o and y_partial must be 16-byte aligned");
  if (M == 0) return ok();
  tpk::GemmProblem p;
  memset(&p, 0, sizeof(p));
  p.A = static_cast<const uint16_t*>(y_fused);
  p.lda = K;
  p.B = static_cast<const uint16_t*>(w_o);
  p.ldb = K;
  p.M = (int)M;
  p.N = (int)E;
  p.K = (int)K;
  p.ep.C = y_partial;
  p.ep.ldc = E;
  p.ep.act = TP_ACT_NONE;
  p.ep.out_f32 = 1;
  p.ep.accumulate = accumulate;
  return hip_status(tpk::launch_gemm(p, tune.tile, tune.path, as_stream(stream)), "tp_o_wo_partial launch");
}

int rmsnorm_rows(const void* x, int64_t M, int64_t K, const void* scale, float eps, void* xnorm_out, void* workspace,
                 size_t workspace_bytes, void* stream) {
  if (x == nullptr || xnorm_out == nullptr || workspace == nullptr)
    return fail(TP_ERR_INVALID_ARG, "x, xnorm_out and workspace must be non-NULL");
  if (M < 0 || K < 1) return fail(TP_ERR_INVALID_ARG, "M = %lld must be >= 0 and K = %lld >= 1", (long long)M,
                                  (long long)K);
  if (M > INT_MAX || K > INT_MAX) return fail(TP_ERR_UNSUPPORTED, "sizes must fit in 31 bits");
  if (K % 8) return fail(TP_ERR_UNSUPPORTED, "K = %lld must be a multiple of 8", (long long)K);
  if (!(eps >= 0.0f) || isinf(eps)) return fail(TP_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (!aligned(x, 16) || !aligned(xnorm_out, 16) || (scale != nullptr && !aligned(scale, 16)))
    return fail(TP_ERR_UNSUPPORTED, "x, xnorm_out and scale must be 16-byte aligned");
  if (!aligned(workspace, 256)) return fail(TP_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  const size_t need = tp_rmsnorm_workspace_min_bytes(M, K);
  if (workspace_bytes < need)
    return fail(TP_ERR_SHAPE, "workspace has %zu bytes, at least %zu needed", workspace_bytes, need);
  if (M == 0) return ok();
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  float* r = reinterpret_cast<float*>(ws);
  uint16_t* t = reinterpret_cast<uint16_t*>(ws + align_up((size_t)M * 4, 256));
  return hip_status(tpk::launch_rmsnorm_rows(static_cast<const uint16_t*>(x), (int)M, (int)K,
                                             static_cast<const uint16_t*>(scale), eps, r, scale ? t : nullptr,
                                             static_cast<uint16_t*>(xnorm_out), as_stream(stream)),
                    "rmsnorm rows launch");
}

int rmsnorm_column_linear(const void* x, int64_t M, int64_t K, const void* scale, float eps, void* xnorm_out,
                          const void* w_shard, const void* bias_shard, const int64_t* subparam_sizes, int n_sub,
                          int tp_size, int rank, void* y, int y_dtype, int layout, int64_t ldy, void* workspace,
                          size_t workspace_bytes, void* stream, const Tuning& tune) {
  tpk::GemmProblem p;
  int st = prepare_column(x, M, K, w_shard, bias_shard, subparam_sizes, n_sub, tp_size, rank, TP_ACT_NONE, y, y_dtype,
                          layout, ldy, &p);
  if (st != TP_OK) return st;
  if (!(eps >= 0.0f) || isinf(eps)) return fail(TP_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (scale != nullptr && !aligned(scale, 16)) return fail(TP_ERR_UNSUPPORTED, "scale must be 16-byte aligned");
  if (xnorm_out != nullptr && !aligned(xnorm_out, 16))
    return fail(TP_ERR_UNSUPPORTED, "xnorm_out must be 16-byte aligned");
  if (workspace == nullptr && M > 0) return fail(TP_ERR_INVALID_ARG, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(TP_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  const size_t need = tp_rmsnorm_workspace_min_bytes(M, K);
  if (workspace_bytes < need)
    return fail(TP_ERR_SHAPE, "workspace has %zu bytes, at least %zu needed", workspace_bytes, need);
  if (M == 0) return ok();

  // Workspace: r [M] f32 | t [K] bf16 | (fast path) the normalised rows [M, K] bf16.
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  float* r = reinterpret_cast<float*>(ws);
  uint16_t* t = reinterpret_cast<uint16_t*>(ws + align_up((size_t)M * 4, 256));
  uint16_t* rows = xnorm_out != nullptr ? static_cast<uint16_t*>(xnorm_out)
                   : workspace_bytes >= tp_rmsnorm_workspace_bytes(M, K) ? reinterpret_cast<uint16_t*>(ws + need)
                                                                         : nullptr;
  hipStream_t s = as_stream(stream);
  hipError_t e = tpk::launch_rmsnorm_rows(static_cast<const uint16_t*>(x), (int)M, (int)K,
                                          static_cast<const uint16_t*>(scale), eps, r, scale ? t : nullptr, rows, s);
  if (e != hipSuccess) return hip_status(e, "rmsnorm statistics launch");
  if (rows != nullptr) {
    // Normalised rows materialised: the GEMM reads them as a plain A (direct-to-LDS loop).
    p.A = rows;
  } else {
    // Fused: the GEMM normalises A while staging it (r per row, t per column).
    p.row_r = r;
    p.col_t = scale ? t : nullptr;
  }
  return hip_status(tpk::launch_gemm(p, tune.tile, tune.path, s), "rmsnorm_column_linear GEMM launch");
}

int lm_head_shard_argmax(const void* x, int64_t B, int64_t K, int64_t vocab, int tp_size, int rank,
                         int64_t max_rows_per_chunk, const void* w_shard, int w_dtype, const float* w_block_scale,
                         float* logits, int32_t* argmax_local, float* max_logit, void* workspace,
                         size_t workspace_bytes, void* stream, const Tuning& tune) {
  if (tp_size < 1) return fail(TP_ERR_INVALID_ARG, "tp_size = %d must be >= 1", tp_size);
  if (rank < 0 || rank >= tp_size) return fail(TP_ERR_INVALID_ARG, "rank %d outside [0, %d)", rank, tp_size);
  if (x == nullptr || w_shard == nullptr || logits == nullptr || argmax_local == nullptr || workspace == nullptr)
    return fail(TP_ERR_INVALID_ARG, "x, w_shard, logits, argmax_local and workspace must be non-NULL");
  if (B < 1 || K < 1 || vocab < 1)
    return fail(TP_ERR_INVALID_ARG, "B = %lld, K = %lld, vocab = %lld must be positive", (long long)B, (long long)K,
                (long long)vocab);
  if (vocab < tp_size) return fail(TP_ERR_SHAPE, "vocab %lld is smaller than tp_size %d", (long long)vocab, tp_size);
  if (B > INT_MAX || K > INT_MAX || vocab > INT_MAX) return fail(TP_ERR_UNSUPPORTED, "sizes must fit in 31 bits");
  if (max_rows_per_chunk < 1)
    return fail(TP_ERR_SHAPE, "max_rows_per_chunk = %lld must be positive", (long long)max_rows_per_chunk);
  if (w_dtype != TP_DTYPE_BF16 && w_dtype != TP_DTYPE_FP8_E4M3)
    return fail(TP_ERR_UNSUPPORTED, "w_dtype %d: the weight must be bf16 or fp8 e4m3", w_dtype);
  if (K % 8) return fail(TP_ERR_UNSUPPORTED, "K = %lld must be a multiple of 8", (long long)K);
  if (w_dtype == TP_DTYPE_FP8_E4M3) {
    if (K % 128) return fail(TP_ERR_UNSUPPORTED, "fp8 weights need K (%lld) a multiple of 128", (long long)K);
    if (w_block_scale == nullptr) return fail(TP_ERR_INVALID_ARG, "fp8 weights need w_block_scale");
    if (!aligned(w_block_scale, 4)) return fail(TP_ERR_UNSUPPORTED, "w_block_scale misaligned");
  }
  if (!aligned(x, 16) || !aligned(w_shard, 16) || !aligned(logits, 4) || !aligned(argmax_local, 4) ||
      (max_logit != nullptr && !aligned(max_logit, 4)))
    return fail(TP_ERR_UNSUPPORTED, "x and w_shard must be 16-byte aligned, outputs 4-byte aligned");
  if (!aligned(workspace, 256)) return fail(TP_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  const int64_t V_r = width_of(vocab, tp_size, rank);
  const int64_t chunk = max_rows_per_chunk < V_r ? max_rows_per_chunk : V_r;
  const size_t need = tpk::lm_head_shape_workspace_bytes(tune.lm_shape, (int)B, (int)V_r, (int)K,
                                                        w_dtype == TP_DTYPE_FP8_E4M3, (int)chunk);
  if (workspace_bytes < need) return fail(TP_ERR_SHAPE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);

  tpk::LmHeadProblem p;
  p.x = static_cast<const uint16_t*>(x);
  p.w = w_shard;
  p.wscale = w_dtype == TP_DTYPE_FP8_E4M3 ? w_block_scale : nullptr;
  p.w_fp8 = w_dtype == TP_DTYPE_FP8_E4M3;
  p.B = (int)B;
  p.K = (int)K;
  p.V = (int)V_r;
  p.chunk = (int)chunk;
  p.logits = logits;
  p.argmax = argmax_local;
  p.maxval = max_logit;
  p.workspace = workspace;
  return hip_status(tpk::launch_lm_head(p, tune.lm_shape, as_stream(stream)), "lm_head_shard_argmax launch");
}

}  // namespace tpabi

extern "C" {

TP_API const char* tp_last_error(void) { return g_err; }

TP_API const char* tp_version(void) { return "tpshard 0.1 gfx950"; }

TP_API int tp_shard_widths(const int64_t* subparam_sizes, int n_sub, int tp_size, int rank, int64_t* width,
                    int64_t* logical_off, int64_t* local_off, int64_t* shard_total) {
  Shard sh;
  int st = resolve_shard(subparam_sizes, n_sub, tp_size, rank, &sh);
  if (st != TP_OK) return st;
  for (int i = 0; i < n_sub; ++i) {
    if (width) width[i] = sh.width[i];
    if (logical_off) logical_off[i] = sh.logical_off[i];
    if (local_off) local_off[i] = sh.local_off[i];
  }
  if (shard_total) *shard_total = sh.total;
  return ok();
}

TP_API int tp_column_linear(const void* x, int64_t M, int64_t K, const void* w_shard, const void* bias_shard,
                     const int64_t* subparam_sizes, int n_sub, int tp_size, int rank, int act, void* y, int y_dtype,
                     int layout, int64_t ldy, void* stream) {
  return tpabi::column_linear(x, M, K, w_shard, bias_shard, subparam_sizes, n_sub, tp_size, rank, act, y, y_dtype,
                              layout, ldy, stream, tpabi::Tuning{});
}

TP_API int tp_quantize_rows_e4m3(const void* x, int64_t M, int64_t K, void* q, float* scale, void* stream) {
  if (M < 0 || K <= 0) return fail(TP_ERR_INVALID_ARG, "M = %lld, K = %lld: need M >= 0, K > 0", (long long)M, (long long)K);
  if (M > 0 && (x == nullptr || q == nullptr || scale == nullptr))
    return fail(TP_ERR_INVALID_ARG, "x, q and scale must be non-NULL");
  if (M > INT_MAX || K > INT_MAX) return fail(TP_ERR_UNSUPPORTED, "M and K must fit in 31 bits");
  if (K % 8) return fail(TP_ERR_UNSUPPORTED, "K = %lld must be a multiple of 8", (long long)K);
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scale, 4))
    return fail(TP_ERR_UNSUPPORTED, "x and q must be 16-byte aligned, scale 4-byte aligned");
  if (M == 0) return ok();
  return hip_status(tpk::launch_quantize_rows_e4m3(static_cast<const uint16_t*>(x), (int)M, (int)K,
                                                   static_cast<uint8_t*>(q), scale, as_stream(stream)),
                    "tp_quantize_rows_e4m3 launch");
}

TP_API int tp_column_linear_fp8(const void* x_q, const float* x_scale, int64_t M, int64_t K, const void* w_q,
                                const float* w_scale, const void* bias_shard, const int64_t* subparam_sizes, int n_sub,
                                int tp_size, int rank, int act, void* y, int y_dtype, int layout, int64_t ldy,
                                void* stream) {
  return tpabi::column_linear_fp8(x_q, x_scale, M, K, w_q, w_scale, bias_shard, subparam_sizes, n_sub, tp_size, rank,
                                  act, y, y_dtype, layout, ldy, stream, tpabi::Tuning{});
}

TP_API int tp_vocab_embedding(const int32_t* tokens, int64_t n_tokens, int64_t vocab, int tp_size, int rank,
                              const void* table_shard, int64_t E, void* out, void* stream) {
  if (tp_size < 1) return fail(TP_ERR_INVALID_ARG, "tp_size = %d must be >= 1", tp_size);
  if (rank < 0 || rank >= tp_size) return fail(TP_ERR_INVALID_ARG, "rank %d outside [0, %d)", rank, tp_size);
  if (n_tokens < 0 || vocab < 1 || E < 1)
    return fail(TP_ERR_INVALID_ARG, "n_tokens = %lld, vocab = %lld, E = %lld: need n_tokens >= 0, vocab > 0, E > 0",
                (long long)n_tokens, (long long)vocab, (long long)E);
  if (table_shard == nullptr || (n_tokens > 0 && (tokens == nullptr || out == nullptr)))
    return fail(TP_ERR_INVALID_ARG, "tokens, table_shard and out must be non-NULL");
  if (vocab < tp_size) return fail(TP_ERR_SHAPE, "vocab %lld is smaller than tp_size %d", (long long)vocab, tp_size);
  if (n_tokens > INT_MAX || vocab > INT_MAX || E > INT_MAX) return fail(TP_ERR_UNSUPPORTED, "sizes must fit in 31 bits");
  if (E % 8) return fail(TP_ERR_UNSUPPORTED, "E = %lld must be a multiple of 8", (long long)E);
  if (!aligned(table_shard, 16) || !aligned(out, 16) || !aligned(tokens, 4))
    return fail(TP_ERR_UNSUPPORTED, "table_shard and out must be 16-byte aligned, tokens 4-byte aligned");
  if (n_tokens == 0) return ok();
  const int64_t rows = width_of(vocab, tp_size, rank);
  int64_t off = 0;
  for (int q = 0; q < rank; ++q) off += width_of(vocab, tp_size, q);
  return hip_status(tpk::launch_embed_shard(tokens, (int)n_tokens, (int)vocab, (int)rows, (int)off,
                                            static_cast<const uint16_t*>(table_shard), (int)E,
                                            static_cast<uint16_t*>(out), as_stream(stream)),
                    "tp_vocab_embedding launch");
}

TP_API int tp_row_linear_partial(const void* x_shard, int64_t M, int64_t K_logical, int64_t N, const void* w_shard,
                          const void* bias, int tp_size, int rank, float* y_partial, int accumulate, void* stream) {
  return tpabi::row_linear_partial(x_shard, M, K_logical, N, w_shard, bias, tp_size, rank, y_partial, accumulate,
                                   stream, tpabi::Tuning{});
}

TP_API int tp_qwi_swiglu(const void* xnorm, int64_t M, int64_t E, int64_t heads, int64_t padded_heads, int64_t qkv,
                         int64_t ff, int tp_size, int rank, const void* w_qwi, void* q, void* y_fused, void* stream) {
  return tpabi::qwi_swiglu(xnorm, M, E, heads, padded_heads, qkv, ff, tp_size, rank, w_qwi, q, y_fused, stream,
                           tpabi::Tuning{});
}

TP_API int tp_o_wo_partial(const void* y_fused, int64_t M, int64_t heads, int64_t padded_heads, int64_t qkv,
                           int64_t ff, int64_t E, int tp_size, int rank, const void* w_o, float* y_partial,
                           int accumulate, void* stream) {
  return tpabi::o_wo_partial(y_fused, M, heads, padded_heads, qkv, ff, E, tp_size, rank, w_o, y_partial, accumulate,
                             stream, tpabi::Tuning{});
}

TP_API int tp_reduce_scatter_residual(const float* const* partials, int tp_size, int64_t batch, int64_t seq,
                                      int64_t N, int dest_rank, const void* residual, void* z, float* y_sum,
                                      void* stream) {
  if (tp_size < 1 || tp_size > TP_MAX_RANKS)
    return fail(TP_ERR_INVALID_ARG, "tp_size = %d outside [1, %d]", tp_size, TP_MAX_RANKS);
  if (dest_rank < 0 || dest_rank >= tp_size)
    return fail(TP_ERR_INVALID_ARG, "dest_rank %d outside [0, %d)", dest_rank, tp_size);
  if (batch < 0 || seq < 1 || N < 1)
    return fail(TP_ERR_INVALID_ARG, "batch = %lld, seq = %lld, N = %lld: need batch >= 0, seq > 0, N > 0",
                (long long)batch, (long long)seq, (long long)N);
  if (partials == nullptr) return fail(TP_ERR_INVALID_ARG, "partials is NULL");
  if (batch > 0 && z == nullptr && y_sum == nullptr) return fail(TP_ERR_INVALID_ARG, "z and y_sum are both NULL");
  if (seq % tp_size)
    return fail(TP_ERR_SHAPE, "seq = %lld does not split evenly over tp_size %d", (long long)seq, tp_size);
  if (N % 4) return fail(TP_ERR_UNSUPPORTED, "N = %lld must be a multiple of 4", (long long)N);
  if (batch > INT_MAX || seq > INT_MAX || N > INT_MAX) return fail(TP_ERR_UNSUPPORTED, "sizes must fit in 31 bits");
  for (int r = 0; r < tp_size; ++r) {
    if (partials[r] == nullptr && batch > 0) return fail(TP_ERR_INVALID_ARG, "partials[%d] is NULL", r);
    if (!aligned(partials[r], 16)) return fail(TP_ERR_UNSUPPORTED, "partials[%d] must be 16-byte aligned", r);
  }
  if (!aligned(residual, 16) || !aligned(z, 16) || !aligned(y_sum, 16))
    return fail(TP_ERR_UNSUPPORTED, "residual, z and y_sum must be 16-byte aligned");
  if (batch == 0) return ok();
  // one thread per four outputs in a 1-D grid of 256-thread workgroups (checked without overflow)
  if (batch * (seq / tp_size) > (int64_t)INT_MAX * 256 / (N / 4))
    return fail(TP_ERR_UNSUPPORTED, "batch * seq / tp_size * N is too large for one launch");
  tpk::ReduceScatterProblem p;
  memset(&p, 0, sizeof(p));
  for (int r = 0; r < tp_size; ++r) p.part[r] = partials[r];
  p.tp = tp_size;
  p.dest = dest_rank;
  p.seq = seq;
  p.sl = seq / tp_size;
  p.N = N;
  p.chunks = batch * p.sl * (N / 4);
  p.residual = static_cast<const uint16_t*>(residual);
  p.z = static_cast<uint16_t*>(z);
  p.y_sum = y_sum;
  return hip_status(tpk::launch_reduce_scatter(p, as_stream(stream)), "tp_reduce_scatter_residual launch");
}

TP_API size_t tp_rmsnorm_workspace_min_bytes(int64_t M, int64_t K) {
  if (M < 0 || K < 0) return 0;
  return align_up((size_t)M * sizeof(float), 256) + align_up((size_t)K * sizeof(uint16_t), 256);
}

TP_API size_t tp_rmsnorm_workspace_bytes(int64_t M, int64_t K) {
  if (M < 0 || K < 0) return 0;
  return tp_rmsnorm_workspace_min_bytes(M, K) + align_up((size_t)M * (size_t)K * sizeof(uint16_t), 256);
}

TP_API int rmsnorm_column_linear(const void* x, int64_t M, int64_t K, const void* scale, float eps, void* xnorm_out,
                                 const void* w_shard, const void* bias_shard, const int64_t* subparam_sizes, int n_sub,
                                 int tp_size, int rank, void* y, int y_dtype, int layout, int64_t ldy, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return tpabi::rmsnorm_column_linear(x, M, K, scale, eps, xnorm_out, w_shard, bias_shard, subparam_sizes, n_sub,
                                      tp_size, rank, y, y_dtype, layout, ldy, workspace, workspace_bytes, stream,
                                      tpabi::Tuning{});
}

TP_API size_t tp_lm_head_workspace_bytes(int64_t B, int64_t vocab, int tp_size, int rank) {
  if (B < 1 || vocab < 1 || tp_size < 1 || rank < 0 || rank >= tp_size || vocab < tp_size || vocab > INT_MAX) return 0;
  return tpk::lm_head_workspace_bytes((int)width_of(vocab, tp_size, rank));
}

TP_API int lm_head_shard_argmax(const void* x, int64_t B, int64_t K, int64_t vocab, int tp_size, int rank,
                         int64_t max_rows_per_chunk, const void* w_shard, int w_dtype, const float* w_block_scale,
                         float* logits, int32_t* argmax_local, float* max_logit, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return tpabi::lm_head_shard_argmax(x, B, K, vocab, tp_size, rank, max_rows_per_chunk, w_shard, w_dtype, w_block_scale,
                                     logits, argmax_local, max_logit, workspace, workspace_bytes, stream,
                                     tpabi::Tuning{});
}

TP_API int lm_head_shard_argmax_noalloc(const void* x, int64_t B, int64_t K, int64_t vocab, int tp_size, int rank,
                                        int64_t max_rows_per_chunk, const void* w_shard, int w_dtype,
                                        const float* w_block_scale, float* logits, int32_t* argmax_local,
                                        float* max_logit, void* stream) {
  // the sizes are checked by the shared body; the scratch must hold this call's candidates
  if (B >= 1 && B <= INT_MAX && K >= 1 && K <= INT_MAX && vocab >= 1 && vocab <= INT_MAX && tp_size >= 1 &&
      rank >= 0 && rank < tp_size && vocab >= tp_size && max_rows_per_chunk >= 1) {
    const int64_t V_r = width_of(vocab, tp_size, rank);
    const int64_t chunk = max_rows_per_chunk < V_r ? max_rows_per_chunk : V_r;
    const size_t need = tpk::lm_head_shape_workspace_bytes(-1, (int)B, (int)V_r, (int)K, w_dtype == TP_DTYPE_FP8_E4M3,
                                                          (int)chunk);
    void* ws = nullptr;
    size_t cap = 0;
    const hipError_t e = tpk::lm_head_scratch(&ws, &cap);
    if (e != hipSuccess) return hip_status(e, "lm_head_shard_argmax_noalloc scratch address");
    if (need > cap)
      return fail(TP_ERR_SHAPE, "the shard's %lld rows need %zu bytes of scratch; the library holds %zu per GPU",
                  (long long)V_r, need, cap);
    return tpabi::lm_head_shard_argmax(x, B, K, vocab, tp_size, rank, max_rows_per_chunk, w_shard, w_dtype,
                                       w_block_scale, logits, argmax_local, max_logit, ws, cap, stream,
                                       tpabi::Tuning{});
  }
  // invalid sizes: the shared body reports them before it looks at the workspace (a stand-in
  // address of zero bytes, never dereferenced: a zero-byte workspace fails its size check)
  return tpabi::lm_head_shard_argmax(x, B, K, vocab, tp_size, rank, max_rows_per_chunk, w_shard, w_dtype,
                                     w_block_scale, logits, argmax_local, max_logit, reinterpret_cast<void*>(256), 0,
                                     stream, tpabi::Tuning{});
}

}  // extern "C"
