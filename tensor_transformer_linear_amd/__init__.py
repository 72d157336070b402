"""Python binding of libtpshard: one tensor-parallel rank's transformer linear layers on MI355X.

Argument marshalling only. Every step of the hot path runs in the library's gfx950 kernels.
The C ABI sees plain pointers and sizes, so this module checks what only the tensors know:
dtype, contiguity, device and the shapes the call implies (the shard widths come from the
library's own ``tp_shard_widths``). A bad call raises ``ValueError`` before anything reaches
the library; a non-zero status from the library raises ``TpError``. PyTorch provides device
memory and streams.

bf16 tensors are ``torch.bfloat16`` (or ``torch.int16``/``uint16`` views of the same bits);
E4M3 tensors are ``torch.uint8`` (or ``torch.float8_e4m3fn``) codes.

``tuning(tile=..., path=..., lm_shape=...)`` (or ``set_gemm_tile`` / ``set_gemm_path`` /
``set_lm_head_shape``) routes the calling thread's calls to the separate tuning library, whose
variants force a GEMM tile, a GEMM main loop or an LM-head launch shape (tests and measurements;
the product library has no such switch). With every choice automatic the calls go to the
product library.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtpshard.so")
TUNING_LIB_PATH = os.path.join(_HERE, "libtpshard_tuning.so")

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
    "tp_lm_head_workspace_bytes": (_sz, [_i64, _i64, _int, _int]),
    "lm_head_shard_argmax": (_int, [_vp, _i64, _i64, _i64, _int, _int, _i64, _vp, _int, _vp, _vp, _vp, _vp, _vp,
                                    _sz, _vp]),
    "lm_head_shard_argmax_noalloc": (_int, [_vp, _i64, _i64, _i64, _int, _int, _i64, _vp, _int, _vp, _vp, _vp, _vp,
                                            _vp]),
    "tp_last_error": (ctypes.c_char_p, []),
    "tp_version": (ctypes.c_char_p, []),
}

# The tuning library's variants (csrc/tpshard_tuning.h): a product entry point's arguments
# followed by the launch choices it takes.
TUNING_CHOICES = {
    "tp_column_linear": ("tile", "path"),
    "tp_column_linear_fp8": ("tile",),
    "tp_row_linear_partial": ("tile", "path"),
    "tp_qwi_swiglu": ("tile", "path"),
    "tp_o_wo_partial": ("tile", "path"),
    "rmsnorm_column_linear": ("tile", "path"),
    "lm_head_shard_argmax": ("lm_shape",),
}


def _tuning_name(name: str) -> str:
    return "tpt_" + (name[3:] if name.startswith("tp_") else name)


TUNING_SIGNATURES = {
    **{_tuning_name(n): (SIGNATURES[n][0], SIGNATURES[n][1] + [_int] * len(c)) for n, c in TUNING_CHOICES.items()},
    "tpt_gemm_pick_tile": (_int, [_i64, _i64, _i64]),
    "tpt_gemm_fp8_pick_tile": (_int, [_i64, _i64, _i64]),
    "tpt_lm_head_shape_count": (_int, []),
    "tpt_mfma_row_sums": (_int, [_int, _vp, _vp, _vp, _vp]),
    "tpt_rmsnorm_rows": (_int, [_vp, _i64, _i64, _vp, ctypes.c_float, _vp, _vp, _sz, _vp]),
    "tpt_stream_probe": (_int, [_int, _int, _vp, _i64, _vp, _vp]),
    "tpt_mfma_rate": (_int, [_int, _int, _int, _vp, _vp]),
    "tp_last_error": (ctypes.c_char_p, []),
}


class TpError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"tpshard status {status}: {message}")
        self.status = status
        self.message = message


_libs: dict = {}


def _load(path: str, sigs: dict) -> ctypes.CDLL:
    if path not in _libs:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
        l = ctypes.CDLL(path)
        for name, (res, args) in sigs.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _libs[path] = l
    return _libs[path]


def lib() -> ctypes.CDLL:
    """The loaded product library. Raises if it has not been built: there is no fallback path."""
    return _load(LIB_PATH, SIGNATURES)


def tuning_lib() -> ctypes.CDLL:
    """The tuning library (the product entry points with forced launch choices)."""
    return _load(TUNING_LIB_PATH, TUNING_SIGNATURES)


_tls = threading.local()
_AUTO = {"tile": -1, "path": -1, "lm_shape": -1}


def _set_choice(**kw) -> None:
    choices = dict(getattr(_tls, "choices", None) or _AUTO)
    choices.update({k: int(v) for k, v in kw.items()})
    _tls.choices = None if choices == _AUTO else choices


@contextlib.contextmanager
def tuning(tile: int = -1, path: int = -1, lm_shape: int = -1):
    """Inside the block, this thread's calls force the given launch choices (-1 = automatic):
    ``tile`` a key of ``GEMM_TILES``, ``path`` one of ``GEMM_PATH_*``, ``lm_shape`` a key of
    ``LM_HEAD_SHAPES``. Calls go to the tuning library, which rejects unknown choices."""
    prev = getattr(_tls, "choices", None)
    _tls.choices = None
    _set_choice(tile=tile, path=path, lm_shape=lm_shape)
    try:
        yield
    finally:
        _tls.choices = prev


def set_gemm_tile(tile: int) -> None:
    """From now on, this thread's GEMM calls force tile ``tile`` (-1 = automatic)."""
    _set_choice(tile=tile)


def set_gemm_path(path: int) -> None:
    """From now on, this thread's GEMM calls force main loop ``path`` (-1 = automatic)."""
    _set_choice(path=path)


def set_lm_head_shape(shape: int) -> None:
    """From now on, this thread's LM-head calls force launch shape ``shape`` (-1 = default)."""
    _set_choice(lm_shape=shape)


def _call(name: str, *args) -> None:
    choices = getattr(_tls, "choices", None)
    if choices is None or name not in TUNING_CHOICES:
        l, status = lib(), getattr(lib(), name)(*args)
    else:
        l = tuning_lib()
        status = getattr(l, _tuning_name(name))(*args, *[choices[c] for c in TUNING_CHOICES[name]])
    if status != TP_OK:
        raise TpError(status, l.tp_last_error().decode())


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


# --- argument checks on the tensors (the C ABI cannot see sizes, dtypes or devices) ---------

_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_E4M3 = (torch.uint8, torch.float8_e4m3fn)


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _tensor(t, name: str, dtypes, shape=None, contiguous: bool = True):
    """``t`` has one of ``dtypes``, is contiguous (if asked) and has ``shape`` (``None`` entries
    are free; ``shape`` may also be a total element count given as an int)."""
    _need(isinstance(t, torch.Tensor), f"{name} must be a torch.Tensor")
    _need(t.dtype in dtypes, f"{name} has dtype {t.dtype}, expected one of {[str(d) for d in dtypes]}")
    if contiguous:
        _need(t.is_contiguous(), f"{name} must be contiguous")
    if isinstance(shape, int):
        _need(t.numel() == shape, f"{name} has {t.numel()} elements, expected {shape}")
    elif shape is not None:
        ok = t.dim() == len(shape) and all(w is None or int(s) == int(w) for s, w in zip(t.shape, shape))
        _need(ok, f"{name} has shape {tuple(t.shape)}, expected {tuple('*' if w is None else w for w in shape)}")


def _same_gpu(**tensors) -> torch.device:
    devs = {n: t.device for n, t in tensors.items() if t is not None}
    first = next(iter(devs.values()))
    for n, d in devs.items():
        _need(d.type == "cuda", f"{n} is on {d}: every tensor must be on the GPU")
        _need(d == first, f"{n} is on {d}, not on {first} with the other tensors")
    return first


def _output_rows(y, name: str, dtypes, M: int, width: int, ldy):
    """An output written as M rows of ``width`` elements at row pitch ``ldy``: returns ``ldy``."""
    _tensor(y, name, dtypes, contiguous=False)
    _need(y.dim() == 2 and y.stride(1) == 1, f"{name} must be 2-D with contiguous rows")
    if ldy is None:
        ldy = y.stride(0)
    _need(int(ldy) == y.stride(0), f"ldy = {ldy} differs from {name}'s row stride {y.stride(0)}")
    _need(y.shape[0] == M and y.shape[1] >= width, f"{name} has shape {tuple(y.shape)}, needs ({M}, >= {width})")
    return int(ldy)


def _shard_total(subparam_sizes, tp_size, rank) -> tuple[int, int]:
    """(rank's shard rows, logical width) from the library's own shard arithmetic."""
    _, _, _, total = tp_shard_widths(subparam_sizes, tp_size, rank)
    return total, sum(int(s) for s in subparam_sizes)


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


def _column_output(y, dev, M, n_r, n_logical, y_dtype, layout, ldy):
    """Checks a given column output (before the device check, so shape errors are reported
    first) or, with ``dev`` set, allocates one; returns ``(y, ldy)``."""
    width = n_r if layout == TP_LAYOUT_LOCAL else n_logical
    dt = torch.bfloat16 if y_dtype == TP_DTYPE_BF16 else torch.float32
    if y is None:
        if dev is None:
            return None, ldy
        y = (torch.empty if layout == TP_LAYOUT_LOCAL else torch.zeros)((M, width), dtype=dt, device=dev)
    ldy = _output_rows(y, "y", _BF16 if y_dtype == TP_DTYPE_BF16 else (torch.float32,), M, width, ldy)
    return y, ldy


def tp_column_linear(x, w_shard, bias_shard, subparam_sizes, tp_size, rank, act=TP_ACT_NONE, y=None,
                     y_dtype=TP_DTYPE_BF16, layout=TP_LAYOUT_LOCAL, ldy=None, stream=None):
    """``y = act(x @ w_shard.T + bias_shard)`` for the rank's column shard; returns ``y``."""
    _tensor(x, "x", _BF16, (None, None))
    M, K = x.shape
    n_r, n_logical = _shard_total(subparam_sizes, tp_size, rank)
    _tensor(w_shard, "w_shard", _BF16, (n_r, K))
    if bias_shard is not None:
        _tensor(bias_shard, "bias_shard", _BF16, (n_r,))
    _column_output(y, None, M, n_r, n_logical, y_dtype, layout, ldy)
    dev = _same_gpu(x=x, w_shard=w_shard, bias_shard=bias_shard, y=y)
    y, ldy = _column_output(y, dev, M, n_r, n_logical, y_dtype, layout, ldy)
    sizes, n = _i64_array(subparam_sizes)
    _call("tp_column_linear", _ptr(x), M, K, _ptr(w_shard), _ptr(bias_shard), sizes, n, tp_size, rank, act, _ptr(y),
          y_dtype, layout, ldy, _stream(stream))
    return y


def tp_vocab_embedding(tokens, vocab, tp_size, rank, table_shard, out=None, stream=None):
    """The rank's embedding rows of int32 ``tokens`` (zero rows outside its vocab shard); returns ``out``."""
    _tensor(tokens, "tokens", (torch.int32,))
    n = tokens.numel()
    v_r, _ = _shard_total([vocab], tp_size, rank)
    _tensor(table_shard, "table_shard", _BF16, (v_r, None))
    E = table_shard.shape[1]
    if out is not None:
        _tensor(out, "out", _BF16, (n, E))
    dev = _same_gpu(tokens=tokens, table_shard=table_shard, out=out)
    if out is None:
        out = torch.empty((n, E), dtype=torch.bfloat16, device=dev)
    _call("tp_vocab_embedding", _ptr(tokens), n, vocab, tp_size, rank, _ptr(table_shard), E, _ptr(out),
          _stream(stream))
    return out


def tp_quantize_rows_e4m3(x, q=None, scale=None, stream=None):
    """Per-row E4M3 codes of bf16 ``x`` and their float32 scales; returns ``(q uint8, scale f32)``."""
    _tensor(x, "x", _BF16, (None, None))
    M, K = x.shape
    if q is not None:
        _tensor(q, "q", _E4M3, (M, K))
    if scale is not None:
        _tensor(scale, "scale", (torch.float32,), (M,))
    dev = _same_gpu(x=x, q=q, scale=scale)
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=dev)
    if scale is None:
        scale = torch.empty((M,), dtype=torch.float32, device=dev)
    _call("tp_quantize_rows_e4m3", _ptr(x), M, K, _ptr(q), _ptr(scale), _stream(stream))
    return q, scale


def tp_column_linear_fp8(x_q, x_scale, w_q, w_scale, bias_shard, subparam_sizes, tp_size, rank, act=TP_ACT_NONE,
                         y=None, y_dtype=TP_DTYPE_BF16, layout=TP_LAYOUT_LOCAL, ldy=None, stream=None):
    """``tp_column_linear`` on E4M3 codes: ``act(x_scale * w_scale * (x_q @ w_q.T) + bias)``; returns ``y``."""
    _tensor(x_q, "x_q", _E4M3, (None, None))
    M, K = x_q.shape
    n_r, n_logical = _shard_total(subparam_sizes, tp_size, rank)
    _tensor(x_scale, "x_scale", (torch.float32,), (M,))
    _tensor(w_q, "w_q", _E4M3, (n_r, K))
    _tensor(w_scale, "w_scale", (torch.float32,), (n_r,))
    if bias_shard is not None:
        _tensor(bias_shard, "bias_shard", _BF16, (n_r,))
    _column_output(y, None, M, n_r, n_logical, y_dtype, layout, ldy)
    dev = _same_gpu(x_q=x_q, x_scale=x_scale, w_q=w_q, w_scale=w_scale, bias_shard=bias_shard, y=y)
    y, ldy = _column_output(y, dev, M, n_r, n_logical, y_dtype, layout, ldy)
    sizes, n = _i64_array(subparam_sizes)
    _call("tp_column_linear_fp8", _ptr(x_q), _ptr(x_scale), M, K, _ptr(w_q), _ptr(w_scale), _ptr(bias_shard), sizes,
          n, tp_size, rank, act, _ptr(y), y_dtype, layout, ldy, _stream(stream))
    return y


def tp_row_linear_partial(x_shard, K_logical, w_shard, bias, tp_size, rank, y_partial=None, accumulate=0,
                          stream=None):
    """The rank's float32 partial ``x_shard @ w_shard.T`` (+ bias on rank 0); returns ``y_partial``."""
    k_r, _ = _shard_total([K_logical], tp_size, rank)
    _tensor(x_shard, "x_shard", _BF16, (None, k_r))
    _tensor(w_shard, "w_shard", _BF16, (None, k_r))
    M, N = x_shard.shape[0], w_shard.shape[0]
    if bias is not None:
        _tensor(bias, "bias", _BF16, (N,))
    if y_partial is not None:
        _tensor(y_partial, "y_partial", (torch.float32,), (M, N))
    dev = _same_gpu(x_shard=x_shard, w_shard=w_shard, bias=bias, y_partial=y_partial)
    if y_partial is None:
        y_partial = torch.empty((M, N), dtype=torch.float32, device=dev)
    _call("tp_row_linear_partial", _ptr(x_shard), M, K_logical, N, _ptr(w_shard), _ptr(bias), tp_size, rank,
          _ptr(y_partial), accumulate, _stream(stream))
    return y_partial


def _head_dims(heads, padded_heads, qkv, ff, tp_size):
    """(h_r, fph, qph, fused) when the sizes are valid, else None (the library then reports why)."""
    if tp_size < 1 or heads < 1 or heads % tp_size or not 0 <= padded_heads < heads or qkv < 1 or ff < 1:
        return None
    fph = ff // (heads - padded_heads)
    return (heads // tp_size, fph, qkv + 2 * fph, qkv + fph) if fph >= 1 else None


def tp_qwi_swiglu(xnorm, heads, padded_heads, qkv, ff, tp_size, rank, w_qwi, y_fused, q=None, stream=None):
    """The rank's fused q_wi projection: SwiGLU of its MLP columns into the MLP slots of
    ``y_fused`` ``[M, h_r, qkv + fph]`` (attention slots untouched) and, when ``q`` is given,
    the query columns ``[M, h_r, qkv]``; returns ``(q, y_fused)``."""
    _tensor(xnorm, "xnorm", _BF16, (None, None))
    M, E = xnorm.shape
    d = _head_dims(heads, padded_heads, qkv, ff, tp_size)
    if d is not None:
        h_r, _, qph, fused = d
        _tensor(w_qwi, "w_qwi", _BF16, (h_r * qph, E))
        _tensor(y_fused, "y_fused", _BF16, M * h_r * fused)
        if q is not None:
            _tensor(q, "q", _BF16, M * h_r * qkv)
    _same_gpu(xnorm=xnorm, w_qwi=w_qwi, y_fused=y_fused, q=q)
    _call("tp_qwi_swiglu", _ptr(xnorm), M, E, heads, padded_heads, qkv, ff, tp_size, rank, _ptr(w_qwi), _ptr(q),
          _ptr(y_fused), _stream(stream))
    return q, y_fused


def tp_o_wo_partial(y_fused, heads, padded_heads, qkv, ff, tp_size, rank, w_o, y_partial=None, accumulate=0,
                    stream=None):
    """The rank's float32 partial of the fused attention-out + MLP-out projection
    ``y_fused [M, h_r (qkv + fph)] @ w_o.T`` with ``w_o [E, h_r (qkv + fph)]``; returns ``y_partial``."""
    _tensor(w_o, "w_o", _BF16, (None, None))
    M, E = y_fused.shape[0], w_o.shape[0]
    d = _head_dims(heads, padded_heads, qkv, ff, tp_size)
    if d is not None:
        h_r, _, _, fused = d
        _tensor(y_fused, "y_fused", _BF16, M * h_r * fused)
        _tensor(w_o, "w_o", _BF16, (E, h_r * fused))
    if y_partial is not None:
        _tensor(y_partial, "y_partial", (torch.float32,), (M, E))
    dev = _same_gpu(y_fused=y_fused, w_o=w_o, y_partial=y_partial)
    if y_partial is None:
        y_partial = torch.empty((M, E), dtype=torch.float32, device=dev)
    _call("tp_o_wo_partial", _ptr(y_fused), M, heads, padded_heads, qkv, ff, E, tp_size, rank, _ptr(w_o),
          _ptr(y_partial), accumulate, _stream(stream))
    return y_partial


def tp_reduce_scatter_residual(partials, batch, seq, dest_rank, residual=None, z=None, y_sum=None, stream=None):
    """Rank ``dest_rank``'s rows of the sequence-parallel reduce-scatter of the float32
    ``partials`` (one ``[batch * seq, N]`` tensor per rank), summed in rank order, plus the bf16
    ``residual``: fills ``z`` (bf16) and/or ``y_sum`` (f32), ``[batch * seq / tp, N]``; returns
    ``(z, y_sum)``."""
    tp = len(partials)
    _need(tp >= 1, "partials must hold one tensor per rank")
    N = partials[0].shape[-1]
    for r, p in enumerate(partials):
        _tensor(p, f"partials[{r}]", (torch.float32,), (batch * seq, N))
    rows = batch * (seq // tp) if seq % tp == 0 else None
    if rows is not None:
        for name, t, dts in (("residual", residual, _BF16), ("z", z, _BF16), ("y_sum", y_sum, (torch.float32,))):
            if t is not None:
                _tensor(t, name, dts, (rows, N))
    _same_gpu(residual=residual, z=z, y_sum=y_sum, **{f"partials[{r}]": p for r, p in enumerate(partials)})
    ptrs = (ctypes.c_void_p * max(1, tp))(*[p.data_ptr() for p in partials])
    _call("tp_reduce_scatter_residual", ctypes.cast(ptrs, ctypes.c_void_p), tp, batch, seq, N, dest_rank,
          _ptr(residual), _ptr(z), _ptr(y_sum), _stream(stream))
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
    _tensor(x, "x", _BF16, (None, None))
    M, K = x.shape
    n_r, n_logical = _shard_total(subparam_sizes, tp_size, rank)
    if scale is not None:
        _tensor(scale, "scale", _BF16, (K,))
    if xnorm_out is not None:
        _tensor(xnorm_out, "xnorm_out", _BF16, (M, K))
    _tensor(w_shard, "w_shard", _BF16, (n_r, K))
    if bias_shard is not None:
        _tensor(bias_shard, "bias_shard", _BF16, (n_r,))
    if workspace is not None:
        _tensor(workspace, "workspace", (torch.uint8,))
    _column_output(y, None, M, n_r, n_logical, y_dtype, layout, ldy)
    dev = _same_gpu(x=x, scale=scale, xnorm_out=xnorm_out, w_shard=w_shard, bias_shard=bias_shard, y=y,
                    workspace=workspace)
    y, ldy = _column_output(y, dev, M, n_r, n_logical, y_dtype, layout, ldy)
    if workspace is None:
        workspace = torch.empty(max(1, tp_rmsnorm_workspace_bytes(M, K)), dtype=torch.uint8, device=dev)
    sizes, n = _i64_array(subparam_sizes)
    _call("rmsnorm_column_linear", _ptr(x), M, K, _ptr(scale), float(eps), _ptr(xnorm_out), _ptr(w_shard),
          _ptr(bias_shard), sizes, n, tp_size, rank, _ptr(y), y_dtype, layout, ldy, _ptr(workspace),
          workspace.numel(), _stream(stream))
    return y


def rmsnorm_rows(x, scale, eps, xnorm_out, workspace, stream=None):
    """The RMSNorm pass of ``rmsnorm_column_linear`` alone, into ``xnorm_out`` (tuning library;
    for measurements that time the column GEMM as the full call runs it)."""
    _tensor(x, "x", _BF16, (None, None))
    M, K = x.shape
    if scale is not None:
        _tensor(scale, "scale", _BF16, (K,))
    _tensor(xnorm_out, "xnorm_out", _BF16, (M, K))
    _tensor(workspace, "workspace", (torch.uint8,))
    _same_gpu(x=x, scale=scale, xnorm_out=xnorm_out, workspace=workspace)
    l = tuning_lib()
    st = l.tpt_rmsnorm_rows(_ptr(x), M, K, _ptr(scale), float(eps), _ptr(xnorm_out), _ptr(workspace),
                            workspace.numel(), _stream(stream))
    if st != TP_OK:
        raise TpError(st, l.tp_last_error().decode())
    return xnorm_out


def tp_lm_head_workspace_bytes(B, vocab, tp_size, rank) -> int:
    return int(lib().tp_lm_head_workspace_bytes(B, vocab, tp_size, rank))


def lm_head_workspace(B, vocab, tp_size, rank, device="cuda"):
    """A workspace for ``lm_head_shard_argmax`` (scratch; zeroed here only for tidiness)."""
    n = tp_lm_head_workspace_bytes(B, vocab, tp_size, rank)
    if n == 0:
        raise TpError(TP_ERR_INVALID_ARG, "invalid LM-head workspace query")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def lm_head_shard_argmax(x, vocab, tp_size, rank, max_rows_per_chunk, w_shard, w_dtype=TP_DTYPE_BF16,
                         w_block_scale=None, logits=None, argmax_local=None, max_logit=None, workspace=None,
                         stream=None):
    """float32 logits of the rank's vocab shard and the per-row local argmax; returns (logits, idx, max)."""
    _tensor(x, "x", _BF16, (None, None))
    B, K = x.shape
    v_r, _ = _shard_total([vocab], tp_size, rank)
    _tensor(w_shard, "w_shard", _E4M3 if w_dtype == TP_DTYPE_FP8_E4M3 else _BF16, (v_r, K))
    if w_block_scale is not None:
        _tensor(w_block_scale, "w_block_scale", (torch.float32,), (v_r, K // 128))
    for name, t, shape, dts in (("logits", logits, (B, v_r), (torch.float32,)),
                                ("argmax_local", argmax_local, (B,), (torch.int32,)),
                                ("max_logit", max_logit, (B,), (torch.float32,)),
                                ("workspace", workspace, None, (torch.uint8,))):
        if t is not None:
            _tensor(t, name, dts, shape)
    dev = _same_gpu(x=x, w_shard=w_shard, w_block_scale=w_block_scale, logits=logits, argmax_local=argmax_local,
                    max_logit=max_logit, workspace=workspace)
    if logits is None:
        logits = torch.empty((B, v_r), dtype=torch.float32, device=dev)
    if argmax_local is None:
        argmax_local = torch.empty((B,), dtype=torch.int32, device=dev)
    if max_logit is None:
        max_logit = torch.empty((B,), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = lm_head_workspace(B, vocab, tp_size, rank, dev)
    _call("lm_head_shard_argmax", _ptr(x), B, K, vocab, tp_size, rank, max_rows_per_chunk, _ptr(w_shard), w_dtype,
          _ptr(w_block_scale), _ptr(logits), _ptr(argmax_local), _ptr(max_logit), _ptr(workspace),
          workspace.numel(), _stream(stream))
    return logits, argmax_local, max_logit


def lm_head_shard_argmax_noalloc(x, vocab, tp_size, rank, max_rows_per_chunk, w_shard, w_dtype=TP_DTYPE_BF16,
                                 w_block_scale=None, logits=None, argmax_local=None, max_logit=None, stream=None):
    """``lm_head_shard_argmax`` with the library's own device scratch instead of a workspace (for
    callers that cannot allocate: pass every output); returns (logits, idx, max)."""
    _tensor(x, "x", _BF16, (None, None))
    B, K = x.shape
    v_r, _ = _shard_total([vocab], tp_size, rank)
    _tensor(w_shard, "w_shard", _E4M3 if w_dtype == TP_DTYPE_FP8_E4M3 else _BF16, (v_r, K))
    if w_block_scale is not None:
        _tensor(w_block_scale, "w_block_scale", (torch.float32,), (v_r, K // 128))
    for name, t, shape, dts in (("logits", logits, (B, v_r), (torch.float32,)),
                                ("argmax_local", argmax_local, (B,), (torch.int32,)),
                                ("max_logit", max_logit, (B,), (torch.float32,))):
        if t is not None:
            _tensor(t, name, dts, shape)
    dev = _same_gpu(x=x, w_shard=w_shard, w_block_scale=w_block_scale, logits=logits, argmax_local=argmax_local,
                    max_logit=max_logit)
    if logits is None:
        logits = torch.empty((B, v_r), dtype=torch.float32, device=dev)
    if argmax_local is None:
        argmax_local = torch.empty((B,), dtype=torch.int32, device=dev)
    _call("lm_head_shard_argmax_noalloc", _ptr(x), B, K, vocab, tp_size, rank, max_rows_per_chunk, _ptr(w_shard),
          w_dtype, _ptr(w_block_scale), _ptr(logits), _ptr(argmax_local), _ptr(max_logit), _stream(stream))
    return logits, argmax_local, max_logit


GEMM_PATH_AUTO, GEMM_PATH_REGISTER, GEMM_PATH_DMA = -1, 0, 1

LM_HEAD_SHAPES = {0: (4, 8, 8, 1), 1: (2, 8, 8, 1), 2: (4, 4, 8, 1), 3: (2, 4, 8, 1), 4: (4, 8, 4, 1),
                  5: (1, 8, 8, 1), 6: (4, 8, 4, 2), 7: (8, 4, 4, 2), 8: ("lds-ring", 64), 9: ("lds-ring", 128),
                  10: ("x-resident", 64), 11: ("row-quad", 0), 12: ("row-quad", 1), 13: ("row-quad", 2),
                  14: ("row-quad", 3), 15: ("row-quad", 4),
                  16: ("row-quad", 5)}


def gemm_pick_tile(M: int, N: int, K: int) -> int:
    """The tile the library picks for an M x N x K bf16 GEMM (a key of ``GEMM_TILES``; -1 if invalid)."""
    return int(tuning_lib().tpt_gemm_pick_tile(M, N, K))


def gemm_fp8_pick_tile(M: int, N: int, K: int) -> int:
    """The tile the library picks for an M x N x K E4M3 GEMM (0 or 2, keys of ``GEMM_TILES``; -1 if invalid)."""
    return int(tuning_lib().tpt_gemm_fp8_pick_tile(M, N, K))


GEMM_TILES = {0: (256, 256), 1: (256, 128), 2: (128, 128), 3: (128, 256), 4: (256, 224), 5: (128, 64), 6: (64, 64)}
