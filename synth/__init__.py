"""Seeded synthetic inputs for the tensor-parallel linear-layer hot path.

This module only *draws* inputs.  It holds none of the method's arithmetic: no
matmul, no GELU, no normalisation, no shard arithmetic.  Both the CPU oracle
(through the tests) and the GPU path consume exactly the arrays it returns, so
a parity test compares the two sides on identical bits.

Storage conventions (what every consumer receives):
  * bf16 tensors are ``numpy.uint16`` arrays of bf16 bit patterns.
  * fp8 tensors are ``numpy.uint8`` arrays of OCP E4M3FN codes.
  * block scales are ``numpy.float32``.

Recipe (per workload and tensor): ``numpy.random.default_rng([2026, cfg, tid])``
draws ``standard_normal`` in float32, multiplies by the stated standard
deviation in float32 and rounds to bf16 with round-to-nearest-even.  Tensor ids:
x = 0, first weight = 1, second weight or bias = 2, RMSNorm scale = 3.

The fp8 weight format of the LM head (Tenstorrent ``lm_head_1d.py``,
``LMHead1DConfig.lm_head_dtype`` stores the projection in an 8-bit block
format) is produced here as a *storage* step: per weight row and per 128-wide
K block, ``scale = amax / 448`` (1.0 for an all-zero block) and
``q = e4m3_rne(w / scale)``, saturating at 448.  Both sides then read the
stored bytes and scales; neither re-derives them.
"""
from __future__ import annotations

import numpy as np

SEED_BASE = 2026
E4M3_MAX = 448.0
FP8_BLOCK = 128

# Tensor ids inside one workload.
TID_X, TID_W1, TID_W2, TID_SCALE = 0, 1, 2, 3


def rng(cfg_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([SEED_BASE, int(cfg_id), int(tensor_id)])


def _f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 bit patterns (nearest, ties to even)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    # no uint32 overflow: the largest non-NaN pattern is 0xFF800000 (-inf)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_normal(shape, std: float, cfg_id: int, tensor_id: int, chunk_rows: int = 4096) -> np.ndarray:
    """bf16 bits of ``std * N(0,1)`` drawn with the workload's seed.

    Large tensors are drawn in row blocks (same generator, consecutive draws) to
    bound the float32 temporary; the result equals one draw of the whole shape.
    """
    shape = tuple(int(s) for s in shape)
    g = rng(cfg_id, tensor_id)
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(shape[0] if len(shape) > 1 else 1, -1)
    rows = flat.shape[0]
    s = np.float32(std)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        z = g.standard_normal((r1 - r0, flat.shape[1]), dtype=np.float32)
        flat[r0:r1] = _f32_to_bf16_bits(z * s)
    return out


def bf16_integers(shape, lo: int, hi: int, seed: int) -> np.ndarray:
    """bf16 bits of uniform integers in [lo, hi] (exact in bf16 for |v| <= 256)."""
    g = np.random.default_rng([SEED_BASE, 9000, int(seed)])
    v = g.integers(lo, hi + 1, size=shape).astype(np.float32)
    return _f32_to_bf16_bits(v)


def bf16_from_float(values) -> np.ndarray:
    """bf16 bits of given float values (used to plant chosen inputs)."""
    return _f32_to_bf16_bits(np.asarray(values, dtype=np.float32))


# --- E4M3FN storage codec used by the weight quantiser (input side only) ----------

def _e4m3_positive_table() -> np.ndarray:
    """Magnitudes of codes 0x00..0x7E of OCP E4M3FN (bias 7, 3 mantissa bits)."""
    vals = np.empty(127, dtype=np.float64)
    for code in range(127):
        e, m = code >> 3, code & 7
        vals[code] = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3_POS = _e4m3_positive_table()


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Nearest E4M3FN code (ties to the even code), saturating to +-448."""
    v = np.asarray(v, dtype=np.float64)
    mag = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, mag, side="left")  # first table value >= mag
    hi = np.clip(hi, 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_lo = mag - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    neg = np.signbit(v) & (code != 0)
    return (code | (neg.astype(np.uint8) << 7)).astype(np.uint8)


def quantize_e4m3_blocks(w_bits: np.ndarray, chunk_rows: int = 2048, block: int = FP8_BLOCK):
    """Per-row, per-``block``-K-block E4M3 storage of a bf16 weight ``[rows, K]``.

    Returns ``(codes uint8 [rows, K], scales float32 [rows, K // block])``.  Rows are
    processed in blocks to bound the temporaries; each row's result is independent.
    """
    rows, k = w_bits.shape
    if k % block:
        raise ValueError(f"K={k} must be a multiple of {block}")
    q = np.empty((rows, k), dtype=np.uint8)
    scale = np.empty((rows, k // block), dtype=np.float32)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        w = (w_bits[r0:r1].astype(np.uint32) << 16).view(np.float32).reshape(r1 - r0, k // block, block)
        amax = np.abs(w).max(axis=2)
        s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
        q[r0:r1] = e4m3_encode((w / s[:, :, None]).astype(np.float32)).reshape(r1 - r0, k)
        scale[r0:r1] = s
    return q, scale


def quantize_e4m3_channels(w_bits: np.ndarray, chunk_rows: int = 2048):
    """Per-output-channel E4M3 storage of a bf16 weight ``[rows, K]``: one scale per row
    (``amax / 448`` over the row).  Returns ``(codes uint8 [rows, K], scales float32 [rows])``."""
    q, s = quantize_e4m3_blocks(w_bits, chunk_rows, block=w_bits.shape[1])
    return q, s[:, 0].copy()


# --- The five workloads, as shapes and distributions ---------------------------------

WORKLOADS = {
    1: dict(name="gpt2-small MLP shard, tp=2, ranks 0 and 1",
            batch=2, seq=128, hidden=768, inter=3072, tp=2, w_std=0.02),
    2: dict(name="fused-QKV GQA column shard, tp=8 rank 0",
            batch=4, seq=1024, hidden=4096, sizes=(4096, 1024, 1024), tp=8, rank=0, w_std=0.02),
    3: dict(name="llama-8B MLP shard, tp=8",
            batch=8, seq=1024, hidden=4096, inter=14336, tp=8, rank=0, w_std=0.02),
    4: dict(name="RMSNorm prologue into column GEMM, tp=8",
            batch=16, seq=2048, hidden=8192, out_logical=24576, tp=8, rank=0, w_std=0.02,
            scale_std=0.1, eps=1e-6),
    5: dict(name="vocab-sharded decode LM head, tp=8 rank 0",
            batch=32, hidden=4096, vocab=128256, tp=8, rank=0, chunk=4008, w_std=0.02),
}


def workload_inputs(cfg_id: int, rows: int | None = None) -> dict:
    """Inputs of one workload at its full size (or its first ``rows`` x-rows).

    Shard weights are drawn directly at the shard shape the workload states
    (configs 3-5 give shards); configs 1 and 2 give logical weights, which the
    caller slices into shards with the shard arithmetic under test.
    """
    c = WORKLOADS[cfg_id]
    out = {}
    m_full = c["batch"] * c.get("seq", 1)
    m = m_full if rows is None else min(rows, m_full)
    x = bf16_normal((m_full, c["hidden"]), 1.0, cfg_id, TID_X) if rows is None else \
        _first_rows_normal(m, c["hidden"], 1.0, cfg_id, TID_X)
    out["x"] = x
    if cfg_id == 1:
        out["w_fc"] = bf16_normal((c["inter"], c["hidden"]), c["w_std"], cfg_id, TID_W1)
        out["w_proj"] = bf16_normal((c["hidden"], c["inter"]), c["w_std"], cfg_id, TID_W2)
    elif cfg_id == 2:
        n_log = sum(c["sizes"])
        out["w"] = bf16_normal((n_log, c["hidden"]), c["w_std"], cfg_id, TID_W1)
        out["bias"] = bf16_normal((n_log,), c["w_std"], cfg_id, TID_W2)
    elif cfg_id == 3:
        shard = c["inter"] // c["tp"]
        out["w_fc"] = bf16_normal((shard, c["hidden"]), c["w_std"], cfg_id, TID_W1)
        out["w_proj"] = bf16_normal((c["hidden"], shard), c["w_std"], cfg_id, TID_W2)
    elif cfg_id == 4:
        shard = c["out_logical"] // c["tp"]
        out["w"] = bf16_normal((shard, c["hidden"]), c["w_std"], cfg_id, TID_W1)
        out["scale"] = bf16_normal((c["hidden"],), c["scale_std"], cfg_id, TID_SCALE)
    elif cfg_id == 5:
        shard = c["vocab"] // c["tp"]
        w = bf16_normal((shard, c["hidden"]), c["w_std"], cfg_id, TID_W1)
        out["w"] = w
        out["w_fp8"], out["w_scale"] = quantize_e4m3_blocks(w)
    return out


def _first_rows_normal(rows: int, cols: int, std: float, cfg_id: int, tensor_id: int) -> np.ndarray:
    """The first ``rows`` rows of ``bf16_normal((M, cols), ...)`` without drawing all M."""
    g = rng(cfg_id, tensor_id)
    z = g.standard_normal((rows, cols), dtype=np.float32)
    return _f32_to_bf16_bits(z * np.float32(std))
