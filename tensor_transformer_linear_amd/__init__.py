"""Python binding of libtpshard: one tensor-parallel rank's transformer linear layers on MI355X.

Argument marshalling only. Every step of the hot path runs in the library's
gfx950 kernels; this module checks nothing the library does not check itself,
passes ``data_ptr()`` and the current HIP stream, and turns a non-zero status
into ``TpError``. PyTorch provides device memory and streams.

bf16 tensors are ``torch.bfloat16`` (or ``torch.int16``/``uint16`` views of the same
bits); fp8 weights are ``torch.uint8`` (or ``torch.float8_e4m3fn``) codes.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtpshard.so")

TP_OK, TP_ERR_INVALID_ARG, TP_ERR_SHAPE, TP_ERR_UNSUPPORTED, TP_ERR_HIP = range(5)
TP_DTYPE_BF16, TP_DTYPE_F32, TP_DTYPE_FP8_E4M3 = 0, 1, 2
TP_ACT_NONE, TP_ACT_GELU_ERF = 0, 1
TP_LAYOUT_LOCAL, TP_LAYOUT_LOGICAL = 0, 1
TP_MAX_SUBPARAMS = 16

# Exported symbols and their C signatures, as declared in include/tpshard.h.
_i64, _int, _vp, _sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
_P64 = ctypes.POINTER(ctypes.c_int64)
SIGNATURES = {
    "tp_shard_widths": (_int, [_P64, _int, _int, _int, _P64, _P64, _P64, _P64]),
    "tp_column_linear": (_int, [_vp, _i64, _i64, _vp, _vp, _P64, _int, _int, _int, _int, _vp, _int, _int, _i64, _vp]),
    "tp_row_linear_partial": (_int, [_vp, _i64, _i64, _i64, _vp, _vp, _int, _int, _vp, _int, _vp]),
    "tp_quantize_rows_e4m3": (_int, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "tp_vocab_embedding": (_int, [_vp, _i64, _i64, _int, _int, _vp, _i64, _vp, _vp]),
    "tp_column_linear_fp8": (_int, [_vp, _vp, _i64, _i64, _vp, _vp, _vp, _P64, _int, _int, _int, _int, _vp, _int,
                                    _int, _i64, _vp]),
    "tp_qwi_swiglu": (_int, [_vp, _i64, _i64, _i64, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp, _vp]),
    "tp_o_wo_partial": (_int, [_vp, _i64, _i64, _i64, _i64, _i64, _i64, _int, _int, _vp, _vp, _int, _vp]),
    "tp_reduce_scatter_residual": (_int, [_vp, _int, _i64, _i64, _i64, _int, _vp, _vp, _vp, _vp]),
    "tp_rmsnorm_workspace_bytes": (_sz, [_i64, _i64]),
    "tp_rmsnorm_workspace_min_bytes": (_sz, [_i64, _i64]),
    "rmsnorm_column_linear": (_int, [_vp, _i64, _i64, _vp, ctypes.c_float, _vp, _vp, _vp, _P64, _int, _int, _int,
                                     _vp, _int, _int, _i64, _vp, _sz, _vp]),
    "tp_lm_head_workspace_bytes": (_sz, [_i64, _i64, _int, _int, _i64]),
    "lm_head_shard_argmax": (_int, [_vp, _i64, _i64, _i64, _int, _int, _i64, _vp, _int, _vp, _vp, _vp, _vp, _vp,
                                    _sz, _vp]),
    "tp_last_error": (ctypes.c_char_p, []),
    "tp_version": (ctypes.c_char_p, []),
    "tp_debug_set_gemm_tile": (_int, [_int]),
    "tp_debug_set_gemm_path": (_int, [_int]),
    "tp_debug_set_lm_head_shape": (_int, [_int]),
    "tp_debug_gemm_pick_tile": (_int, [_i64, _i64, _i64]),
}


class TpError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"tpshard status {status}: {message}")
        self.status = status
        self.message = message


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library. Raises if it has not been built: there is no fallback path."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def _check(status: int) -> None:
    if status != TP_OK:
        raise TpError(status, lib().tp_last_error().decode())


def _i64_array(vals):
    vals = [int(v) for v in vals]
    return (ctypes.c_int64 * max(1, len(vals)))(*vals), len(vals)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def version() -> str:
    return lib().tp_version().decode()


def tp_shard_widths(subparam_sizes, tp_size: int, rank: int):
    """``(width, logical_off, local_off, shard_total)`` of ``rank``'s shard (host arithmetic)."""
    sizes, n = _i64_array(subparam_sizes)
    w = (ctypes.c_int64 * max(1, n))()
    lo = (ctypes.c_int64 * max(1, n))()
    lc = (ctypes.c_int64 * max(1, n))()
    tot = ctypes.c_int64()
    _check(lib().tp_shard_widths(sizes, n, tp_size, rank, w, lo, lc, ctypes.byref(tot)))
    return list(w[:n]), list(lo[:n]), list(lc[:n]), tot.value


def tp_column_linear(x, w_shard, bias_shard, subparam_sizes, tp_size, rank, act=TP_ACT_NONE, y=None,
                     y_dtype=TP_DTYPE_BF16, layout=TP_LAYOUT_LOCAL, ldy=None, stream=None):
    """``y = act(x @ w_shard.T + bias_shard)`` for the rank's column shard; returns ``y``."""
    M, K = x.shape
    sizes, n = _i64_array(subparam_sizes)
    if y is None:
        width = int(w_shard.shape[0]) if layout == TP_LAYOUT_LOCAL else sum(int(s) for s in subparam_sizes)
        dt = torch.bfloat16 if y_dtype == TP_DTYPE_BF16 else torch.float32
        y = (torch.empty if layout == TP_LAYOUT_LOCAL else torch.zeros)((M, width), dtype=dt, device=x.device)
    if ldy is None:
        ldy = y.stride(0) if y.dim() == 2 else y.shape[-1]
    _check(lib().tp_column_linear(_ptr(x), M, K, _ptr(w_shard), _ptr(bias_shard), sizes, n, tp_size, rank, act,
                                  _ptr(y), y_dtype, layout, ldy, _stream(stream)))
    return y


def tp_vocab_embedding(tokens, vocab, tp_size, rank, table_shard, out=None, stream=None):
    """The rank's embedding rows of int32 ``tokens`` (zero rows outside its vocab shard); returns ``out``."""
    n = tokens.numel()
    E = table_shard.shape[1]
    if out is None:
        out = torch.empty((n, E), dtype=torch.bfloat16, device=table_shard.device)
    _check(lib().tp_vocab_embedding(_ptr(tokens), n, vocab, tp_size, rank, _ptr(table_shard), E, _ptr(out),
                                    _stream(stream)))
    return out


def tp_quantize_rows_e4m3(x, q=None, scale=None, stream=None):
    """Per-row E4M3 codes of bf16 ``x`` and their float32 scales; returns ``(q uint8, scale f32)``."""
    M, K = x.shape
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check(lib().tp_quantize_rows_e4m3(_ptr(x), M, K, _ptr(q), _ptr(scale), _stream(stream)))
    return q, scale


def tp_column_linear_fp8(x_q, x_scale, w_q, w_scale, bias_shard, subparam_sizes, tp_size, rank, act=TP_ACT_NONE,
                         y=None, y_dtype=TP_DTYPE_BF16, layout=TP_LAYOUT_LOCAL, ldy=None, stream=None):
    """``tp_column_linear`` on E4M3 codes: ``act(x_scale * w_scale * (x_q @ w_q.T) + bias)``; returns ``y``."""
    M, K = x_q.shape
    sizes, n = _i64_array(subparam_sizes)
    if y is None:
        width = int(w_q.shape[0]) if layout == TP_LAYOUT_LOCAL else sum(int(s) for s in subparam_sizes)
        dt = torch.bfloat16 if y_dtype == TP_DTYPE_BF16 else torch.float32
        y = (torch.empty if layout == TP_LAYOUT_LOCAL else torch.zeros)((M, width), dtype=dt, device=x_q.device)
    if ldy is None:
        ldy = y.stride(0) if y.dim() == 2 else y.shape[-1]
    _check(lib().tp_column_linear_fp8(_ptr(x_q), _ptr(x_scale), M, K, _ptr(w_q), _ptr(w_scale), _ptr(bias_shard),
                                      sizes, n, tp_size, rank, act, _ptr(y), y_dtype, layout, ldy, _stream(stream)))
    return y


def tp_row_linear_partial(x_shard, K_logical, w_shard, bias, tp_size, rank, y_partial=None, accumulate=0,
                          stream=None):
    """The rank's float32 partial ``x_shard @ w_shard.T`` (+ bias on rank 0); returns ``y_partial``."""
    M = x_shard.shape[0]
    N = w_shard.shape[0]
    if y_partial is None:
        y_partial = torch.empty((M, N), dtype=torch.float32, device=x_shard.device)
    _check(lib().tp_row_linear_partial(_ptr(x_shard), M, K_logical, N, _ptr(w_shard), _ptr(bias), tp_size, rank,
                                       _ptr(y_partial), accumulate, _stream(stream)))
    return y_partial


def tp_qwi_swiglu(xnorm, heads, padded_heads, qkv, ff, tp_size, rank, w_qwi, y_fused, q=None, stream=None):
    """The rank's fused q_wi projection: SwiGLU of its MLP columns into the MLP slots of
    ``y_fused`` ``[M, h_r, qkv + fph]`` (attention slots untouched) and, when ``q`` is given,
    the query columns ``[M, h_r, qkv]``; returns ``(q, y_fused)``."""
    M, E = xnorm.shape
    _check(lib().tp_qwi_swiglu(_ptr(xnorm), M, E, heads, padded_heads, qkv, ff, tp_size, rank, _ptr(w_qwi), _ptr(q),
                               _ptr(y_fused), _stream(stream)))
    return q, y_fused


def tp_o_wo_partial(y_fused, heads, padded_heads, qkv, ff, tp_size, rank, w_o, y_partial=None, accumulate=0,
                    stream=None):
    """The rank's float32 partial of the fused attention-out + MLP-out projection
    ``y_fused [M, h_r (qkv + fph)] @ w_o.T`` with ``w_o [E, h_r (qkv + fph)]``; returns ``y_partial``."""
    M = y_fused.shape[0]
    E = w_o.shape[0]
    if y_partial is None:
        y_partial = torch.empty((M, E), dtype=torch.float32, device=y_fused.device)
    _check(lib().tp_o_wo_partial(_ptr(y_fused), M, heads, padded_heads, qkv, ff, E, tp_size, rank, _ptr(w_o),
                                 _ptr(y_partial), accumulate, _stream(stream)))
    return y_partial


def tp_reduce_scatter_residual(partials, batch, seq, dest_rank, residual=None, z=None, y_sum=None, stream=None):
    """Rank ``dest_rank``'s rows of the sequence-parallel reduce-scatter of the float32
    ``partials`` (one ``[batch * seq, N]`` tensor per rank), summed in rank order, plus the bf16
    ``residual``: fills ``z`` (bf16) and/or ``y_sum`` (f32), ``[batch * seq / tp, N]``; returns
    ``(z, y_sum)``."""
    tp = len(partials)
    N = partials[0].shape[-1]
    ptrs = (ctypes.c_void_p * max(1, tp))(*[p.data_ptr() for p in partials])
    _check(lib().tp_reduce_scatter_residual(ctypes.cast(ptrs, ctypes.c_void_p), tp, batch, seq, N, dest_rank,
                                            _ptr(residual), _ptr(z), _ptr(y_sum), _stream(stream)))
    return z, y_sum


def tp_rmsnorm_workspace_bytes(M: int, K: int) -> int:
    return int(lib().tp_rmsnorm_workspace_bytes(M, K))


def tp_rmsnorm_workspace_min_bytes(M: int, K: int) -> int:
    return int(lib().tp_rmsnorm_workspace_min_bytes(M, K))


def rmsnorm_column_linear(x, scale, eps, w_shard, bias_shard, subparam_sizes, tp_size, rank, xnorm_out=None,
                          y=None, y_dtype=TP_DTYPE_BF16, layout=TP_LAYOUT_LOCAL, ldy=None, workspace=None,
                          stream=None):
    """RMSNorm rows of ``x`` (optionally into ``xnorm_out``), then the rank's column linear; returns ``y``.

    Without ``workspace`` a workspace of ``tp_rmsnorm_workspace_bytes`` (fast, materialised
    path) is allocated; pass one of ``tp_rmsnorm_workspace_min_bytes`` for the fused path."""
    M, K = x.shape
    sizes, n = _i64_array(subparam_sizes)
    if y is None:
        width = int(w_shard.shape[0]) if layout == TP_LAYOUT_LOCAL else sum(int(s) for s in subparam_sizes)
        dt = torch.bfloat16 if y_dtype == TP_DTYPE_BF16 else torch.float32
        y = (torch.empty if layout == TP_LAYOUT_LOCAL else torch.zeros)((M, width), dtype=dt, device=x.device)
    if ldy is None:
        ldy = y.stride(0)
    if workspace is None:
        workspace = torch.empty(max(1, tp_rmsnorm_workspace_bytes(M, K)), dtype=torch.uint8, device=x.device)
    _check(lib().rmsnorm_column_linear(_ptr(x), M, K, _ptr(scale), float(eps), _ptr(xnorm_out), _ptr(w_shard),
                                       _ptr(bias_shard), sizes, n, tp_size, rank, _ptr(y), y_dtype, layout, ldy,
                                       _ptr(workspace), workspace.numel() * workspace.element_size(),
                                       _stream(stream)))
    return y


def tp_lm_head_workspace_bytes(B, vocab, tp_size, rank, max_rows_per_chunk) -> int:
    return int(lib().tp_lm_head_workspace_bytes(B, vocab, tp_size, rank, max_rows_per_chunk))


def lm_head_workspace(B, vocab, tp_size, rank, max_rows_per_chunk, device="cuda"):
    """A workspace for ``lm_head_shard_argmax`` (scratch; zeroed here only for tidiness)."""
    n = tp_lm_head_workspace_bytes(B, vocab, tp_size, rank, max_rows_per_chunk)
    if n == 0:
        raise TpError(TP_ERR_INVALID_ARG, "invalid LM-head workspace query")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def lm_head_shard_argmax(x, vocab, tp_size, rank, max_rows_per_chunk, w_shard, w_dtype=TP_DTYPE_BF16,
                         w_block_scale=None, logits=None, argmax_local=None, max_logit=None, workspace=None,
                         stream=None):
    """float32 logits of the rank's vocab shard and the per-row local argmax; returns (logits, idx, max)."""
    B, K = x.shape
    V_r = int(w_shard.shape[0])
    dev = x.device
    if logits is None:
        logits = torch.empty((B, V_r), dtype=torch.float32, device=dev)
    if argmax_local is None:
        argmax_local = torch.empty((B,), dtype=torch.int32, device=dev)
    if max_logit is None:
        max_logit = torch.empty((B,), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = lm_head_workspace(B, vocab, tp_size, rank, max_rows_per_chunk, dev)
    _check(lib().lm_head_shard_argmax(_ptr(x), B, K, vocab, tp_size, rank, max_rows_per_chunk, _ptr(w_shard),
                                      w_dtype, _ptr(w_block_scale), _ptr(logits), _ptr(argmax_local),
                                      _ptr(max_logit), _ptr(workspace), workspace.numel(), _stream(stream)))
    return logits, argmax_local, max_logit


def set_gemm_tile(tile: int) -> None:
    """Force a GEMM tile configuration on this thread (-1 = automatic); for tests and tuning."""
    _check(lib().tp_debug_set_gemm_tile(tile))


def set_gemm_path(path: int) -> None:
    """Force the GEMM main loop on this thread: -1 automatic, 0 register staging, 1 direct-to-LDS."""
    _check(lib().tp_debug_set_gemm_path(path))


GEMM_PATH_AUTO, GEMM_PATH_REGISTER, GEMM_PATH_DMA = -1, 0, 1


def set_lm_head_shape(shape: int) -> None:
    """Force the LM head's launch shape on this thread (-1 = default); for tests and tuning."""
    _check(lib().tp_debug_set_lm_head_shape(shape))


LM_HEAD_SHAPES = {0: (4, 8, 8, 1), 1: (2, 8, 8, 1), 2: (4, 4, 8, 1), 3: (2, 4, 8, 1), 4: (4, 8, 4, 1),
                  5: (1, 8, 8, 1), 6: (8, 8, 4, 2), 7: (8, 4, 4, 2), 8: ("lds-ring", 64), 9: ("lds-ring", 128)}


def gemm_pick_tile(M: int, N: int, K: int) -> int:
    return int(lib().tp_debug_gemm_pick_tile(M, N, K))


GEMM_TILES = {0: (256, 256), 1: (256, 128), 2: (128, 128), 3: (128, 256), 4: (256, 224), 5: (128, 64), 6: (64, 64)}
