"""CPU oracle for one tensor-parallel rank's share of a transformer block's linear layers.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the bench's
CPU-baseline leg may import this module.  The GPU library never calls it and
shares no code, header, table or constant generator with it.

Everything here is the plain definition of what the hot path computes, written
out in numpy float64 from exactly widened bf16 / E4M3 inputs, then rounded once
where the method rounds.  A library primitive (numpy's float64 matmul, scipy's
double-precision ``erfc``) serves as a step; there is no blocking, fusion or
reordering beyond the definitions.  Sources (web pages):

  [nanotron]  nanotron rules page "Tensor-Parallel Component Patterns",
              sections "Attention Module" and "MLP Module".
  [deepspeed] DeepSpeed ``deepspeed/module_inject/layers.py``, class
              ``SubParamLinearLayer`` (its docstring, ``__init__``, ``forward``).
  [palm]      google-research ``scaling_transformer_inference_efficiency/
              layers/two_d_parallel_xmap.py``: ``allgather_layernorm``,
              ``unembed_manual``, ``transformer_layer_weight_gathered``.
  [tt]        Tenstorrent ``models/common/modules/lm_head/lm_head_1d.py``:
              module docstring, ``LMHead1DConfig``, ``LMHead1D.forward``,
              ``LMHead1D.from_model_args``.
  [cerebras]  "Cerebras Modelzoo Layers" API page, ``Transformer`` parameters.

Notation: ``bf16(v)`` rounds a float32 to bf16 (nearest, ties to even);
``f32(v)`` rounds a float64 to float32 (nearest, ties to even).  Inputs arrive
as bf16 / E4M3 bit patterns (``uint16`` / ``uint8``).  Where the pages leave a
step open, the reading taken is stated at the function.

Parity pins: every function here is checked by the CPU tests against brute
force, closed forms, invariants or library routines (see ``tests/test_oracle_*``).
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erfc as _erfc

RMS_EPS = 1e-6
FP8_BLOCK = 128

ACT_NONE, ACT_GELU = 0, 1
OUT_BF16, OUT_F32 = 0, 1
LAYOUT_LOCAL, LAYOUT_LOGICAL = 0, 1


# --------------------------------------------------------------------------------------
# Codecs
# --------------------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (bf16 is the top half of a float32)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f32(v) -> np.ndarray:
    """Round float64 to float32, nearest-even (numpy's cast)."""
    return np.asarray(v, dtype=np.float64).astype(np.float32)


def bf16_round(v32: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 bit patterns, nearest with ties to even.

    bf16 keeps the top 16 bits of the float32 pattern; the 16 dropped bits are
    compared with half an ulp (0x8000) and ties go to the even kept pattern.
    NaN maps to the quiet NaN 0x7FC0; overflow rounds to infinity as the
    pattern arithmetic carries into the exponent.
    """
    a = np.ascontiguousarray(v32, dtype=np.float32)
    u = a.view(np.uint32)
    keep = (u >> np.uint32(16)).astype(np.uint32)
    rest = u & np.uint32(0xFFFF)
    up = (rest > 0x8000) | ((rest == 0x8000) & ((keep & np.uint32(1)) == 1))
    out = (keep + up.astype(np.uint32)).astype(np.uint16)
    out = np.where(np.isnan(a), np.uint16(0x7FC0), out).astype(np.uint16)
    return out


def e4m3_table() -> np.ndarray:
    """Value of every OCP 8-bit E4M3FN code, from the format's definition.

    Layout s.eeee.mmm with exponent bias 7: a normal code is
    (-1)^s * (1 + m/8) * 2^(e-7); e = 0 gives the subnormals (-1)^s * (m/8) * 2^-6;
    the codes with e = 15 and m = 7 (0x7F, 0xFF) are NaN; there are no infinities,
    so 0x7E = 448 is the largest finite value.  (The page's ``lm_head_dtype``
    is an 8-bit block format; the E4M3FN reading is stated where it is used.)
    """
    t = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            t[code] = np.nan
        elif e == 0:
            t[code] = s * (m / 8.0) * 2.0 ** -6
        else:
            t[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


_E4M3 = e4m3_table()


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


# --------------------------------------------------------------------------------------
# O1 - shard widths  [deepspeed] __init__; [nanotron] local dims; [tt] from_model_args
# --------------------------------------------------------------------------------------

def shard_widths(subparam_sizes, tp_size: int, rank: int):
    """Per-sub-parameter widths and offsets of rank ``rank`` of ``tp_size``.

    [deepspeed] ``SubParamLinearLayer`` views a weight's output dimension as
    several logical sub-parameters (e.g. q, k, v) and partitions *each one*
    separately along the output dimension; the widths are resolved once per
    model.  [nanotron] uses ``n // tp`` for evenly divisible dimensions.

    Reading for a size that ``tp_size`` does not divide (the page gives no body
    for its width function): a balanced split whose remainder goes to the lowest
    ranks, ``w_s(r) = S_s // tp + (r < S_s % tp)``; a sub-parameter smaller than
    ``tp_size`` is rejected.

    Returns ``(width, logical_off, local_off, total)``: lists over sub-params of
    the rank's width, the first logical output row it owns, the first row inside
    the rank's materialised shard, and the shard's total rows.  The shard is the
    concatenation, in sub-parameter order, of the logical row ranges
    ``[logical_off[s], logical_off[s] + width[s])``.
    """
    sizes = [int(s) for s in subparam_sizes]
    if tp_size < 1:
        raise ValueError(f"tp_size must be >= 1, got {tp_size}")
    if not 0 <= rank < tp_size:
        raise ValueError(f"rank {rank} outside [0, {tp_size})")
    if len(sizes) < 1:
        raise ValueError("at least one sub-parameter size is required")
    for s in sizes:
        if s < tp_size:
            raise ValueError(f"sub-parameter size {s} is smaller than tp_size {tp_size}")

    def w(size, r):
        return size // tp_size + (1 if r < size % tp_size else 0)

    width, logical_off, local_off = [], [], []
    base = 0
    local = 0
    for size in sizes:
        width.append(w(size, rank))
        logical_off.append(base + sum(w(size, q) for q in range(rank)))
        local_off.append(local)
        local += width[-1]
        base += size
    return width, logical_off, local_off, local


def shard_rows(subparam_sizes, tp_size: int, rank: int) -> np.ndarray:
    """Logical output rows held by the rank's shard, in shard order."""
    width, loff, _, _ = shard_widths(subparam_sizes, tp_size, rank)
    return np.concatenate([np.arange(o, o + w) for w, o in zip(width, loff)]).astype(np.int64)


def take_column_shard(w_logical: np.ndarray, subparam_sizes, tp_size: int, rank: int) -> np.ndarray:
    """Materialise a rank's column shard (rows of ``[N_logical, K]``), as done once at load."""
    return np.ascontiguousarray(w_logical[shard_rows(subparam_sizes, tp_size, rank)])


def take_row_shard(w_logical: np.ndarray, tp_size: int, rank: int) -> np.ndarray:
    """A rank's row-parallel shard: columns of ``[N, K_logical]`` (the input dim is split)."""
    rows = shard_rows([w_logical.shape[1]], tp_size, rank)
    return np.ascontiguousarray(w_logical[:, rows])


# --------------------------------------------------------------------------------------
# O2 - column-parallel linear  [deepspeed] forward; [nanotron] MLP c_fc + F.gelu
# --------------------------------------------------------------------------------------

def gelu_erf(a32: np.ndarray) -> np.ndarray:
    """Exact (erf) GELU of float32 values in double: a * Phi(a) = 0.5 a (1 + erf(a / sqrt 2)).

    [nanotron] applies ``F.gelu`` between ``c_fc`` and ``c_proj``; ``F.gelu``'s
    default and [cerebras] ``Transformer(activation='gelu')`` are the erf form.
    ``1 + erf(z)`` is evaluated as ``erfc(-z)`` (the same function): the sum
    cancels in float64 for a < -5, where erfc keeps full relative accuracy.
    """
    a = np.asarray(a32, dtype=np.float64)
    return 0.5 * a * _erfc(-a / math.sqrt(2.0))


def linear_sums(x_bits, w_bits, bias_bits=None) -> np.ndarray:
    """The exact sums ``sum_k x[m,k] W[j,k] (+ b[j])`` in float64, before any rounding.

    [deepspeed] ``forward``: ``input @ weight.T`` then ``+ bias``.  Every product of two bf16
    values is exact in float64.  The linear layers below round these sums; the tests use them
    to check that a GPU output one bf16 unit away from the oracle's is a rounding straddle.
    """
    x = bf16_to_f64(x_bits)
    w = bf16_to_f64(w_bits)
    if x.shape[1] != w.shape[1]:
        raise ValueError("x and weight K differ")
    acc = x @ w.T
    if bias_bits is not None:
        b = bf16_to_f64(bias_bits)
        if b.shape != (w.shape[0],):
            raise ValueError(f"bias has {b.size} entries, expected {w.shape[0]}")
        acc = acc + b[None, :]
    return acc


def column_linear(x_bits, w_shard_bits, bias_shard_bits, subparam_sizes, tp_size, rank,
                  act=ACT_NONE, out_dtype=OUT_BF16, layout=LAYOUT_LOCAL, n_logical=None):
    """One rank's column-parallel linear with sub-parameter sharding.

    [deepspeed] forward: ``output = input @ weight.T`` then ``+ bias``, on the
    rank's materialised shard (weight rows and bias entries of the rank's slice
    of every sub-parameter); the input is replicated across ranks.
    [nanotron] ``MLP``: ``c_fc`` output keeps ``intermediate // tp`` columns,
    then ``F.gelu``.

    Per output element: ``acc = sum_k x[m,k] W_r[j,k] + b_r[j]`` (float64), then
    ``a = f32(acc)``; with GELU ``a = f32(gelu(a))`` -- one rounding of the
    fused result to the output type (reading: the activation is applied to the
    float32 accumulator, then rounded once).  Output ``bf16(a)`` (uint16 bits)
    or ``a`` (float32).

    ``layout=LAYOUT_LOCAL`` returns ``[M, N_r]``.  ``LAYOUT_LOGICAL`` returns the
    rank's columns placed at their logical positions in ``[M, n_logical]`` and a
    boolean mask of the columns this rank wrote (the others are untouched).
    """
    width, loff, lcl, total = shard_widths(subparam_sizes, tp_size, rank)
    if np.shape(w_shard_bits)[0] != total:
        raise ValueError(f"weight shard has {np.shape(w_shard_bits)[0]} rows, shard total is {total}")
    a = f32(linear_sums(x_bits, w_shard_bits, bias_shard_bits))
    if act == ACT_GELU:
        a = f32(gelu_erf(a))
    y = bf16_round(a) if out_dtype == OUT_BF16 else a
    if layout == LAYOUT_LOCAL:
        return y
    if n_logical is None:
        n_logical = sum(int(s) for s in subparam_sizes)
    out = np.zeros((y.shape[0], n_logical), dtype=y.dtype)
    mask = np.zeros(n_logical, dtype=bool)
    for wd, lo, lc in zip(width, loff, lcl):
        out[:, lo:lo + wd] = y[:, lc:lc + wd]
        mask[lo:lo + wd] = True
    return out, mask


# --------------------------------------------------------------------------------------
# O3 - row-parallel partial  [nanotron] MLP c_proj / Attention c_proj
# --------------------------------------------------------------------------------------

def row_linear_partial(x_shard_bits, w_shard_bits, bias_bits=None, rank=0, y_prev=None):
    """One rank's row-parallel partial sum, float32, before any reduction.

    [nanotron] ``TensorParallelRowLinear(intermediate, hidden)``: each rank holds
    the input columns ``K_r`` of its shard and the matching weight columns, and
    its product is a partial of the full output; the pages reduce the partials
    with a collective afterwards.  ``P_r[m,n] = f32(sum_{k<K_r} x_r[m,k] W_r[n,k])``.

    Reading for the bias (the pages' row layers use ``bias=False``): only rank 0
    adds it, so that the sum over ranks equals the unsharded output.  With
    ``y_prev`` the partial is added to an existing float32 buffer in one
    rounding: ``f32(y_prev + sum)`` (used to form the rank-ordered sum).
    """
    x = bf16_to_f64(x_shard_bits)
    w = bf16_to_f64(w_shard_bits)
    if x.shape[1] != w.shape[1]:
        raise ValueError("x shard and weight shard K differ")
    acc = x @ w.T
    if bias_bits is not None and rank == 0:
        acc = acc + bf16_to_f64(bias_bits)[None, :]
    if y_prev is not None:
        acc = acc + np.asarray(y_prev, dtype=np.float32).astype(np.float64)
    return f32(acc)


def rank_ordered_sum(partials) -> np.ndarray:
    """``S = f32(f32(P_0 + P_1) + P_2 ...)``: the partials summed in rank order."""
    s = np.asarray(partials[0], dtype=np.float32)
    for p in partials[1:]:
        s = f32(s.astype(np.float64) + np.asarray(p, dtype=np.float32).astype(np.float64))
    return s


def mlp_rank(x_bits, w_fc_shard_bits, w_proj_shard_bits, rank=0, y_prev=None):
    """[nanotron] ``MLP.forward`` for one rank: ``c_fc`` (column) -> GELU -> ``c_proj`` partial.

    GELU is elementwise, so each rank applies it to its own columns and feeds
    ``c_proj`` with no exchange in between.  ``g_r`` is bf16 (the intermediate
    activation dtype), then the row partial is float32.
    """
    n_r = w_fc_shard_bits.shape[0]
    g = column_linear(x_bits, w_fc_shard_bits, None, [n_r], 1, 0, act=ACT_GELU, out_dtype=OUT_BF16)
    return g, row_linear_partial(g, w_proj_shard_bits, None, rank=rank, y_prev=y_prev)


# --------------------------------------------------------------------------------------
# O5 - RMSNorm prologue  [palm] allgather_layernorm, transformer_layer_weight_gathered
# --------------------------------------------------------------------------------------

def rmsnorm_factor(x_bits, eps=RMS_EPS) -> np.ndarray:
    """The exact per-row factor ``1 / sqrt(mean_k x^2 + eps)`` in float64 (before its float32
    rounding): [palm] ``allgather_layernorm``'s ``rsqrt(mean2 + eps)`` over the whole row."""
    x = bf16_to_f64(x_bits)
    ms = np.sum(x * x, axis=1) / x.shape[1]
    return 1.0 / np.sqrt(ms + eps)


def rmsnorm(x_bits, scale_bits=None, eps=RMS_EPS, r=None):
    """bf16 RMS-normalised rows, as the [palm] layer computes them before ``q_wi``.

    Per row: mean of squares in (at least) float32 over the whole hidden
    dimension (one device holds the full row, so the page's cross-shard mean is
    the plain mean); ``r = f32(1 / sqrt(ms + eps))``; ``n = bf16(f32(x * r))``.
    With a learned scale the page adds 1 to the bf16 scale first, so
    ``t = bf16(f32(1 + s))`` and ``y = bf16(n * t)`` (the product of two bf16
    values is exact in float32).  Without a scale (the prefill layer's local
    norm) ``y = n``.  ``r`` (float32 ``[M]``), when given, replaces the computed
    factor: the rows another admissible float32 rounding of the factor gives.
    Returns ``(y_bits uint16 [M, K], r float32 [M])``.
    """
    x = bf16_to_f64(x_bits)
    r = f32(rmsnorm_factor(x_bits, eps)) if r is None else np.asarray(r, dtype=np.float32)
    n = bf16_round(f32(x * r.astype(np.float64)[:, None]))
    if scale_bits is None:
        return n, r
    t = bf16_round(f32(1.0 + bf16_to_f64(scale_bits)))
    y = bf16_round(f32(bf16_to_f64(n) * bf16_to_f64(t)[None, :]))
    return y, r


def rmsnorm_column_linear(x_bits, scale_bits, w_shard_bits, bias_shard_bits, subparam_sizes, tp_size, rank,
                          eps=RMS_EPS, out_dtype=OUT_BF16, layout=LAYOUT_LOCAL, n_logical=None):
    """RMSNorm rows, then the rank's column linear on the bf16 normalised rows.

    Returns ``(y, xnorm_bits)`` where ``y`` is as in ``column_linear``.
    """
    xn, _ = rmsnorm(x_bits, scale_bits, eps)
    y = column_linear(xn, w_shard_bits, bias_shard_bits, subparam_sizes, tp_size, rank,
                      act=ACT_NONE, out_dtype=out_dtype, layout=layout, n_logical=n_logical)
    return y, xn


# --------------------------------------------------------------------------------------
# O6/O7 - vocab-sharded LM head  [tt] LMHead1D; [palm] unembed_manual
# --------------------------------------------------------------------------------------

def lm_head_chunks(v_rows: int, max_rows_per_chunk: int):
    """Chunk sizes and row offsets of a vocab shard of ``v_rows`` rows.

    [tt] ``from_model_args`` splits the output projection into pieces of at most
    ``max_rows_per_chunk`` rows, all full except the last, which holds what is left; the
    pieces sit back to back along the vocab.  So a chunk starts at every multiple of the
    chunk size below ``v_rows`` and runs to the next multiple or to the end of the shard.
    """
    if max_rows_per_chunk <= 0:
        raise ValueError("max_rows_per_chunk must be positive")
    offs = list(range(0, v_rows, max_rows_per_chunk))
    sizes = [min(max_rows_per_chunk, v_rows - o) for o in offs]
    return sizes, offs


def vocab_shard(vocab: int, tp_size: int, rank: int):
    """``(rows, first_vocab_id)`` of the rank's vocab shard (O1 with one sub-parameter)."""
    width, loff, _, _ = shard_widths([vocab], tp_size, rank)
    return width[0], loff[0]


def lm_head_sums(x_bits, w_shard_bits=None, w_fp8=None, w_scale=None, max_rows_per_chunk=None):
    """float64 logits of one vocab shard before their float32 rounding, chunk by chunk,
    concatenated.

    [tt] ``LMHead1D.forward``: one linear per weight split, outputs trimmed to
    their logical widths and concatenated along the vocab dimension; each device
    ends with the complete logits of its vocab shard (no partial sums).

    bf16 weight: ``sum_k x[b,k] W[v,k]``.  E4M3 weight with per-row, per-128-K
    block scales (reading of the page's 8-bit block weight format):
    ``sum_blk s[v,blk] * sum_{k in blk} x[b,k] dec(q[v,k])``.
    """
    x = bf16_to_f64(x_bits)
    if w_shard_bits is not None:
        w = bf16_to_f64(w_shard_bits)
        v_rows = w.shape[0]

        def chunk(lo, hi):
            return x @ w[lo:hi].T
    else:
        q = e4m3_to_f64(w_fp8)
        s = np.asarray(w_scale, dtype=np.float32).astype(np.float64)
        v_rows, k = q.shape
        if k % FP8_BLOCK:
            raise ValueError("fp8 K must be a multiple of 128")
        nb = k // FP8_BLOCK

        def chunk(lo, hi):
            part = np.zeros((x.shape[0], hi - lo))
            for blk in range(nb):
                ks = slice(blk * FP8_BLOCK, (blk + 1) * FP8_BLOCK)
                part += (x[:, ks] @ q[lo:hi, ks].T) * s[lo:hi, blk][None, :]
            return part
    c = v_rows if max_rows_per_chunk is None else max_rows_per_chunk
    sizes, offs = lm_head_chunks(v_rows, c)
    return np.concatenate([chunk(o, o + n) for n, o in zip(sizes, offs)], axis=1)


def lm_head_logits(x_bits, w_shard_bits=None, w_fp8=None, w_scale=None, max_rows_per_chunk=None):
    """float32 logits of one vocab shard: ``f32`` of ``lm_head_sums`` ([palm]
    ``unembed_manual`` computes logits in float32)."""
    return f32(lm_head_sums(x_bits, w_shard_bits, w_fp8, w_scale, max_rows_per_chunk))


def shard_argmax(logits32: np.ndarray):
    """Per row, the lowest local index attaining the maximum logit, and that maximum.

    [tt] leaves the argmax over the gathered shards to the caller; each shard's
    candidate is its own maximum.  Reading: ties go to the lowest index; NaN
    entries are ignored.  Returns ``(idx int32 [B], max float32 [B])``.
    """
    l = np.asarray(logits32, dtype=np.float32)
    clean = np.where(np.isnan(l), -np.inf, l)
    idx = np.argmax(clean, axis=1).astype(np.int32)  # numpy returns the first maximum
    return idx, clean[np.arange(l.shape[0]), idx].astype(np.float32)


def global_argmax(per_rank):
    """Combine per-rank ``(idx, max, vocab_offset)`` triples: largest max, ties to the lowest rank."""
    best_v = None
    best_i = None
    for idx, mx, off in per_rank:
        g = idx.astype(np.int64) + off
        if best_v is None:
            best_v, best_i = mx.copy(), g.copy()
        else:
            better = mx > best_v
            best_v = np.where(better, mx, best_v)
            best_i = np.where(better, g, best_i)
    return best_i, best_v


# --------------------------------------------------------------------------------------
# F1 - fp8 prefill column linear  [palm] transformer_layer_weight_gathered (QuantizedLayer)
# --------------------------------------------------------------------------------------
#
# [palm] multiplies the normalised activations by the quantised ``q_wi`` weights and then
# applies the per-output-channel ``q_wi_scale`` to the matmul result before casting it to
# the intermediate dtype.  Reading taken for a product on fp8 matrix cores: the weights
# are stored as E4M3 codes with one float32 scale per output channel (a storage format,
# produced by the input generator), and the activations are quantised per row (one float32
# scale per token) by the method itself, as defined here; both scales and the bias are
# applied to the exact product.

E4M3_MAX = 448.0

# finite non-negative E4M3 values in increasing order, and their codes
_E4M3_POS_CODES = np.array([c for c in range(0x7F)], dtype=np.uint8)  # 0x00 .. 0x7E
_E4M3_POS_VALS = _E4M3[:0x7F]


def e4m3_encode(v32: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code of float32 values: ties to the code with the even mantissa,
    magnitudes of 448 or more saturate to 448 (the format has no infinity), and the sign
    is the float's sign bit (signed zero).

    Follows the OCP 8-bit definition: every finite E4M3 value is a candidate; the nearest one
    wins; on an exact tie the candidate whose 3-bit mantissa is even (code LSB 0) wins, which
    is round-to-nearest-even on the significand.  NaN inputs are not defined here.
    """
    v = np.asarray(v32, dtype=np.float32).astype(np.float64)
    mag = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS_VALS, mag, side="left")  # first value >= mag
    hi = np.minimum(hi, len(_E4M3_POS_VALS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _E4M3_POS_VALS[lo]
    d_hi = _E4M3_POS_VALS[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((_E4M3_POS_CODES[hi] & 1) == 0))
    code = np.where(pick_hi, _E4M3_POS_CODES[hi], _E4M3_POS_CODES[lo]).astype(np.uint8)
    code = np.where(mag == _E4M3_POS_VALS[hi], _E4M3_POS_CODES[hi], code).astype(np.uint8)
    # the code's sign is the float's sign bit: E4M3 has a signed zero, so -0.0 and negative
    # quotients that round to zero encode as 0x80
    return np.where(np.signbit(v), code | np.uint8(0x80), code).astype(np.uint8)


def quantize_rows_e4m3(x_bits):
    """Per-row (per-token) E4M3 quantisation of bf16 activations.

    Row m: ``s[m] = f32(amax_k |x[m,k]| / 448)`` (1 for an all-zero row), then
    ``q[m,k] = e4m3(f32(x[m,k] / s[m]))`` with both divisions rounded to float32 once
    (nearest even).  The row's largest magnitude maps to 448 up to that rounding; larger
    quotients saturate.  Returns ``(codes uint8 [M,K], scales float32 [M])``.
    """
    x = bf16_to_f64(x_bits).astype(np.float32)
    amax = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    s = (amax.astype(np.float32) / np.float32(E4M3_MAX)).astype(np.float32)
    s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
    q = e4m3_encode((x / s[:, None]).astype(np.float32))
    return q, s


def linear_sums_fp8(xq, x_scale, wq, w_scale, bias_bits=None) -> np.ndarray:
    """``x_scale[m] * w_scale[j] * sum_k dec(xq[m,k]) dec(wq[j,k]) (+ b[j])`` in float64, before
    any rounding (every product of two E4M3 values is exact)."""
    x = e4m3_to_f64(xq)
    w = e4m3_to_f64(wq)
    if x.shape[1] != w.shape[1]:
        raise ValueError("x and weight K differ")
    v = np.asarray(x_scale, np.float64)[:, None] * np.asarray(w_scale, np.float64)[None, :] * (x @ w.T)
    if bias_bits is not None:
        b = bf16_to_f64(bias_bits)
        if b.shape != (w.shape[0],):
            raise ValueError(f"bias has {b.size} entries, expected {w.shape[0]}")
        v = v + b[None, :]
    return v


def column_linear_fp8(xq, x_scale, wq_shard, w_scale_shard, bias_shard_bits, subparam_sizes, tp_size, rank,
                      act=ACT_NONE, out_dtype=OUT_BF16, layout=LAYOUT_LOCAL, n_logical=None):
    """One rank's column-parallel linear on E4M3 activations and weights.

    ``acc = sum_k dec(xq[m,k]) dec(wq[j,k])`` (exact in float64: every product of two E4M3
    values is exact), ``v = x_scale[m] * w_scale[j] * acc + b[j]`` (float64), then as
    ``column_linear``: ``a = f32(v)``, GELU on ``a`` if asked, one rounding to the output
    type, LOCAL or LOGICAL placement of the shard's columns.
    """
    width, loff, lcl, total = shard_widths(subparam_sizes, tp_size, rank)
    if np.shape(wq_shard)[0] != total:
        raise ValueError(f"weight shard has {np.shape(wq_shard)[0]} rows, shard total is {total}")
    a = f32(linear_sums_fp8(xq, x_scale, wq_shard, w_scale_shard, bias_shard_bits))
    if act == ACT_GELU:
        a = f32(gelu_erf(a))
    y = bf16_round(a) if out_dtype == OUT_BF16 else a
    if layout == LAYOUT_LOCAL:
        return y
    if n_logical is None:
        n_logical = sum(int(s) for s in subparam_sizes)
    out = np.zeros((y.shape[0], n_logical), dtype=y.dtype)
    mask = np.zeros(n_logical, dtype=bool)
    for wd, lo, lc in zip(width, loff, lcl):
        out[:, lo:lo + wd] = y[:, lc:lc + wd]
        mask[lo:lo + wd] = True
    return out, mask


# --------------------------------------------------------------------------------------
# F4 - vocab-parallel embedding lookup  [palm] embed_manual
# --------------------------------------------------------------------------------------

def embed_shard(tokens, vocab: int, tp_size: int, rank: int, table_bits):
    """One rank's share of the embedding lookup.

    [palm] ``embed_manual``: each device holds the rows of its vocab shard; a token's id minus
    the shard's first id indexes the table, and tokens outside the shard give a zero row, so
    summing the ranks' outputs (the page's reduce-scatter) yields the full lookup.  Shards
    follow ``vocab_shard`` (the LM head's split).  Reading: ids outside ``[0, vocab)`` give a
    zero row on every rank.  Returns bf16 bits ``[n_tokens, E]``.
    """
    tok = np.asarray(tokens, dtype=np.int64).reshape(-1)
    rows, off = vocab_shard(vocab, tp_size, rank)
    tbl = np.asarray(table_bits, dtype=np.uint16)
    if tbl.shape[0] != rows:
        raise ValueError(f"table has {tbl.shape[0]} rows, the shard has {rows}")
    local = tok - off
    hit = (local >= 0) & (local < rows) & (tok >= 0) & (tok < vocab)
    out = np.zeros((tok.size, tbl.shape[1]), dtype=np.uint16)
    out[hit] = tbl[local[hit]]
    return out


# --------------------------------------------------------------------------------------
# F2 - fused q_wi projection with SwiGLU, fused o_wo row partial
#      [palm] _transformer_layer_weight_stationary, transformer_layer_weight_gathered:
#      the q_wi projection, the SwiGLU step and the o_wo projection
# --------------------------------------------------------------------------------------

def swish(v) -> np.ndarray:
    """Swish with unit slope, ``v * sigmoid(v) = v / (1 + exp(-v))``, in float64.

    [palm] forms the MLP activation as ``swish2(wi0) * wi1`` (SwiGLU, at the full d_ff width
    rather than the 2/3-scaled one).  ``swish2`` is not defined on the page; reading: the Swish
    of the GLU-variants paper that the page cites, with beta = 1 (SiLU).  For v < -709 the
    exponential overflows to inf and the quotient is -0, its limit.
    """
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def qwi_dims(heads: int, padded_heads: int, qkv: int, ff: int, tp_size: int):
    """``(h_r, fph, qph)``: heads per rank, MLP columns per head, q_wi columns per head.

    [palm] slices each head's q_wi output into ``qkv`` query columns, then ``wi0`` and ``wi1``
    of ``ff // (heads - padded_heads)`` columns each: the d_ff width is spread over the real
    heads, and the padded heads (there so the head axis divides the device mesh) carry the
    same per-head width.  Heads are split evenly over ranks (reading: ``heads`` includes the
    padding and must divide by ``tp_size``).
    """
    if heads < 1 or not (0 <= padded_heads < heads) or qkv < 1 or ff < 1 or tp_size < 1:
        raise ValueError("need heads >= 1, 0 <= padded_heads < heads, qkv >= 1, ff >= 1, tp_size >= 1")
    if heads % tp_size:
        raise ValueError(f"heads {heads} do not split evenly over {tp_size} ranks")
    fph = ff // (heads - padded_heads)
    if fph < 1:
        raise ValueError("ff is smaller than the number of real heads")
    return heads // tp_size, fph, qkv + 2 * fph


def qwi_swiglu(x_bits, w_qwi_bits, heads: int, padded_heads: int, qkv: int, ff: int, tp_size: int, rank: int):
    """One rank's fused q_wi projection and the SwiGLU of its MLP columns.

    [palm] q_wi: ``einsum('bte,hed->bthd', xnorm, q_wi)`` over the rank's heads, in the
    intermediate dtype; ``q = q_wi[..., :qkv]``, ``wi0`` and ``wi1`` the next two ``fph``-wide
    slices; SwiGLU: ``y_mlp = swish2(wi0) * wi1``.

    ``w_qwi_bits`` is the rank's weight with the per-head output axis first, E contiguous:
    ``[h_r * qph, E]``, head-major, and within a head ``qkv`` query rows, ``fph`` wi0 rows,
    ``fph`` wi1 rows (the page's ``[heads, embed, q_wi_per_head]`` shard, transposed once at
    load).  Per element: ``q_wi = bf16(f32(sum_e x w))``; ``y = bf16(f32(swish(wi0) * wi1))``
    on the bf16 values of wi0 and wi1 (reading: Swish and the product are evaluated together
    and rounded once).  Returns ``(q [M, h_r, qkv], y_mlp [M, h_r, fph])`` as bf16 bits.
    """
    h_r, fph, qph = qwi_dims(heads, padded_heads, qkv, ff, tp_size)
    if not 0 <= rank < tp_size:
        raise ValueError(f"rank {rank} outside [0, {tp_size})")
    x = bf16_to_f64(x_bits)
    w = bf16_to_f64(w_qwi_bits)
    if w.shape[0] != h_r * qph or w.shape[1] != x.shape[1]:
        raise ValueError(f"w_qwi is {w.shape}, expected ({h_r * qph}, {x.shape[1]})")
    qwi = bf16_round(f32(x @ w.T)).reshape(x.shape[0], h_r, qph)
    q = qwi[:, :, :qkv]
    wi0 = bf16_to_f64(qwi[:, :, qkv:qkv + fph])
    wi1 = bf16_to_f64(qwi[:, :, qkv + fph:])
    y = bf16_round(f32(swish(wi0) * wi1))
    return np.ascontiguousarray(q), y


def fuse_heads(y_att_bits, y_mlp_bits) -> np.ndarray:
    """[palm] ``y_fused = concatenate([y_att, y_mlp], -1)``: per head, the attention output's
    ``qkv`` columns, then the MLP's ``fph`` columns: ``[M, h_r, qkv + fph]``."""
    return np.concatenate([np.asarray(y_att_bits, dtype=np.uint16), np.asarray(y_mlp_bits, dtype=np.uint16)], axis=-1)


def o_wo_partial(y_fused_bits, w_o_bits, y_prev=None) -> np.ndarray:
    """One rank's fused attention-out and MLP-out projection, float32, before any reduction.

    [palm] o_wo: ``einsum('bthd,hde->bte', y_fused, o_wo)`` contracts over the rank's heads
    and each head's ``qkv + fph`` columns; the page then reduce-scatters the partials over the
    devices holding the other heads.  ``w_o_bits`` is ``[E, h_r * (qkv + fph)]`` (the page's
    ``[heads, d, embed]`` shard transposed once at load, so the contraction axis is
    contiguous).  ``P[m, e] = f32(sum_{h,d} y_fused[m,h,d] o_wo[h,d,e])``; the row-parallel
    partial with the flattened (head, d) axis as its input width.
    """
    yf = np.asarray(y_fused_bits, dtype=np.uint16)
    return row_linear_partial(yf.reshape(yf.shape[0], -1), w_o_bits, None, rank=0, y_prev=y_prev)


# --------------------------------------------------------------------------------------
# F3 - sequence-parallel reduce-scatter of row partials, residual add
#      [nanotron] MLP Module (c_proj output [batch, seq // tp, hidden]);
#      [palm] o_wo step (psum_scatter of the partials) and residual step
# --------------------------------------------------------------------------------------

def seq_slice_rows(batch: int, seq: int, tp_size: int, dest: int) -> np.ndarray:
    """Token rows (of the ``[batch * seq]`` axis) that rank ``dest`` holds after a
    sequence-parallel scatter: positions ``[dest * sl, (dest + 1) * sl)`` of every sequence,
    ``sl = seq // tp_size``, in batch-major order.

    [nanotron] the row-parallel ``c_proj`` returns ``[batch_size, seq_length // tp_size,
    hidden_size]``; [palm] scatters the reduced output along the sequence axis in tiles.
    Reading: ``seq`` must divide by ``tp_size`` (the page's ``seq_length // tp_size`` with no
    remainder).
    """
    if tp_size < 1 or not 0 <= dest < tp_size:
        raise ValueError("need tp_size >= 1 and 0 <= dest < tp_size")
    if seq < 1 or seq % tp_size:
        raise ValueError(f"seq {seq} does not split evenly over {tp_size} ranks")
    sl = seq // tp_size
    return (np.arange(batch)[:, None] * seq + dest * sl + np.arange(sl)[None, :]).reshape(-1)


def reduce_scatter_residual(partials, batch: int, seq: int, dest: int, residual_bits=None):
    """Rank ``dest``'s output of the reduce-scatter of the ranks' row partials, plus the residual.

    ``partials[r]`` is rank r's float32 partial ``[batch * seq, N]`` (``row_linear_partial`` or
    ``o_wo_partial``).  ``S = f32(f32(P_0 + P_1) + ...)`` over the rows of ``dest``'s sequence
    slice (reading: the sum runs in rank order in float32, the plainest fixed order for the
    collective the pages leave unspecified); ``z = bf16(f32(S + x))`` with the bf16 residual
    ``x`` of the slice (``[batch * sl, N]``), [palm] ``z = intermediate_dtype(y_out + x)``.
    Returns ``(S, z)``; ``z`` is None without a residual.
    """
    rows = seq_slice_rows(batch, seq, len(partials), dest)
    S = rank_ordered_sum([np.asarray(p, dtype=np.float32)[rows] for p in partials])
    if residual_bits is None:
        return S, None
    r = bf16_to_f64(residual_bits)
    if r.shape != S.shape:
        raise ValueError(f"residual is {r.shape}, the slice is {S.shape}")
    return S, bf16_round(f32(S.astype(np.float64) + r))
