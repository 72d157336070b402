"""Fused q_wi projection with SwiGLU and the fused o_wo partial on the GPU against the oracle.

* Integer inputs whose products and sums are exact in float32 and in bf16: the query columns
  are bit-exact and the SwiGLU outputs may differ only where float32 and float64 evaluation of
  the Swish straddle a bf16 rounding boundary (one ulp, rare). This pins the head map, the
  gate/value pairing and the placement in y_fused, on every tile shape and both main loops.
* Gaussian inputs: max|err| <= 2e-2 rms; wi0 and wi1 are rounded to bf16 before the SwiGLU,
  so an accumulator that straddles a bf16 boundary moves the output by up to two ulps.
* The o_wo partial (float32) and the whole chain q_wi -> SwiGLU -> o_wo.
* The full-size workload (8192 tokens, E 8192, 64 heads of 128, d_ff 32768, tp 8 rank 0),
  checked on sampled rows.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import tensor_transformer_linear_amd as tt
from helpers import TOL, assert_close, dev_bf16, host_bits

pytestmark = pytest.mark.gpu

SENTINEL = 0x3F81  # bf16 1.0078125: marks the attention slots, which must stay untouched


def _run(x, w, heads, padded, qkv, ff, tp, rank, with_q=True):
    h_r, fph, qph = oracle.qwi_dims(heads, padded, qkv, ff, tp)
    M = x.shape[0]
    xd, wd = dev_bf16(x), dev_bf16(w)
    yf = torch.full((M, h_r, qkv + fph), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    q = torch.empty((M, h_r, qkv), dtype=torch.bfloat16, device="cuda") if with_q else None
    tt.tp_qwi_swiglu(xd, heads, padded, qkv, ff, tp, rank, wd, yf, q=q)
    torch.cuda.synchronize()
    yb = host_bits(yf)
    return (host_bits(q) if with_q else None), yb[:, :, qkv:], yb[:, :, :qkv]


def _exact_inputs(M, E, rows, seed):
    x = synth.bf16_integers((M, E), -1, 1, seed)
    w = synth.bf16_integers((rows, E), -1, 1, seed + 1)
    return x, w


def _check_exact(q, y, att, q_ref, y_ref, what):
    assert np.array_equal(q, q_ref), f"{what}: query columns differ"
    assert np.all(att == SENTINEL), f"{what}: attention slots were written"
    d = np.abs(y.astype(np.int32) - y_ref.astype(np.int32))
    same_sign = (y & 0x8000) == (y_ref & 0x8000)
    off = d != 0
    assert np.all(same_sign[off] & (d[off] == 1)), f"{what}: SwiGLU outputs more than one ulp off"
    assert np.count_nonzero(off) <= 1e-3 * y.size + 1, f"{what}: {np.count_nonzero(off)} outputs one ulp off"


SHAPES = [
    # M, E, heads, padded, qkv, ff, tp, rank
    (300, 256, 6, 1, 32, 200, 2, 1),     # fph 40: tiles straddle heads
    (520, 512, 8, 0, 64, 2048, 2, 0),    # fph 256
    (77, 128, 4, 0, 24, 168, 1, 0),      # fph 42: unaligned head pitch, scalar stores
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("tile", [-1, 0, 1, 2, 4, 6])
def test_qwi_swiglu_integer_exact(shape, tile):
    M, E, heads, padded, qkv, ff, tp, rank = shape
    h_r, fph, qph = oracle.qwi_dims(heads, padded, qkv, ff, tp)
    x, w = _exact_inputs(M, E, h_r * qph, 7 * M + E)
    q_ref, y_ref = oracle.qwi_swiglu(x, w, heads, padded, qkv, ff, tp, rank)
    tt.set_gemm_tile(tile)
    try:
        q, y, att = _run(x, w, heads, padded, qkv, ff, tp, rank)
    finally:
        tt.set_gemm_tile(-1)
    _check_exact(q, y, att, q_ref, y_ref, f"tile {tile} {shape}")


@pytest.mark.parametrize("shape", [(37, 40, 2, 0, 3, 10, 1, 0),     # E % 32 != 0: register-staged loop; fph 5
                                   (5, 8, 3, 1, 1, 2, 3, 2)])       # E 8, one query column, fph 1, h_r 1
def test_qwi_swiglu_small_and_register_path(shape):
    M, E, heads, padded, qkv, ff, tp, rank = shape
    h_r, fph, qph = oracle.qwi_dims(heads, padded, qkv, ff, tp)
    x, w = _exact_inputs(M, E, h_r * qph, 13 + E)
    q_ref, y_ref = oracle.qwi_swiglu(x, w, heads, padded, qkv, ff, tp, rank)
    q, y, att = _run(x, w, heads, padded, qkv, ff, tp, rank)
    _check_exact(q, y, att, q_ref, y_ref, f"small {shape}")


@pytest.mark.parametrize("path", [0, 1])
def test_qwi_swiglu_both_main_loops(path):
    M, E, heads, padded, qkv, ff, tp, rank = SHAPES[0]
    h_r, fph, qph = oracle.qwi_dims(heads, padded, qkv, ff, tp)
    x, w = _exact_inputs(M, E, h_r * qph, 11)
    q_ref, y_ref = oracle.qwi_swiglu(x, w, heads, padded, qkv, ff, tp, rank)
    tt.set_gemm_path(path)
    try:
        q, y, att = _run(x, w, heads, padded, qkv, ff, tp, rank)
    finally:
        tt.set_gemm_path(-1)
    _check_exact(q, y, att, q_ref, y_ref, f"path {path}")


def test_qwi_swiglu_without_queries():
    M, E, heads, padded, qkv, ff, tp, rank = SHAPES[1]
    h_r, fph, qph = oracle.qwi_dims(heads, padded, qkv, ff, tp)
    x, w = _exact_inputs(M, E, h_r * qph, 12)
    _, y_ref = oracle.qwi_swiglu(x, w, heads, padded, qkv, ff, tp, rank)
    _, y, att = _run(x, w, heads, padded, qkv, ff, tp, rank, with_q=False)
    assert np.all(att == SENTINEL)
    assert np.count_nonzero(y != y_ref) <= 1e-3 * y.size + 1


@pytest.mark.parametrize("shape", SHAPES[:2])
def test_qwi_swiglu_gaussian(shape):
    M, E, heads, padded, qkv, ff, tp, rank = shape
    h_r, fph, qph = oracle.qwi_dims(heads, padded, qkv, ff, tp)
    x = synth.bf16_normal((M, E), 1.0, 60, 0)
    w = synth.bf16_normal((h_r * qph, E), 0.02, 60, 1)
    q_ref, y_ref = oracle.qwi_swiglu(x, w, heads, padded, qkv, ff, tp, rank)
    q, y, att = _run(x, w, heads, padded, qkv, ff, tp, rank)
    assert np.all(att == SENTINEL)
    assert_close(q, q_ref, what="q")
    assert_close(y, y_ref, what="swiglu", straddle=5e-3, ulps=2)


def test_padded_heads_are_zero():
    M, E, heads, padded, qkv, ff, tp, rank = 64, 128, 4, 2, 16, 96, 2, 1  # rank 1 holds both padded heads
    h_r, fph, qph = oracle.qwi_dims(heads, padded, qkv, ff, tp)
    x = synth.bf16_normal((M, E), 1.0, 61, 0)
    w = np.zeros((h_r * qph, E), dtype=np.uint16)
    q, y, att = _run(x, w, heads, padded, qkv, ff, tp, rank)
    assert not np.any(oracle.bf16_to_f64(q)) and not np.any(oracle.bf16_to_f64(y))


def test_qwi_swiglu_empty():
    w = torch.zeros((112 * 3, 256), dtype=torch.bfloat16, device="cuda")
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    yf = torch.empty((0, 3, 72), dtype=torch.bfloat16, device="cuda")
    tt.tp_qwi_swiglu(x, 6, 1, 32, 200, 2, 1, w, yf)


@pytest.mark.parametrize("tile", [-1, 0, 2])
def test_o_wo_partial(tile):
    M, heads, padded, qkv, ff, tp, E = 300, 6, 1, 32, 200, 2, 264
    h_r, fph, _ = oracle.qwi_dims(heads, padded, qkv, ff, tp)
    yf = synth.bf16_normal((M, h_r, qkv + fph), 1.0, 62, 0)
    w_o = synth.bf16_normal((E, h_r * (qkv + fph)), 0.02, 62, 1)
    ref = oracle.o_wo_partial(yf, w_o)
    tt.set_gemm_tile(tile)
    try:
        out = tt.tp_o_wo_partial(dev_bf16(yf).view(M, -1), heads, padded, qkv, ff, tp, 0, dev_bf16(w_o))
        torch.cuda.synchronize()
    finally:
        tt.set_gemm_tile(-1)
    assert_close(out.cpu().numpy(), ref, tol=1e-4, what="o_wo partial")


def test_o_wo_rank_ordered_sum():
    M, heads, padded, qkv, ff, tp, E = 128, 4, 0, 16, 64, 2, 136  # fph 16
    h_r, fph, _ = oracle.qwi_dims(heads, padded, qkv, ff, tp)
    d = qkv + fph
    yf = synth.bf16_normal((M, heads, d), 1.0, 63, 0)
    w_o = synth.bf16_normal((E, heads * d), 0.02, 63, 1)
    out = torch.empty((M, E), dtype=torch.float32, device="cuda")
    parts = []
    for r in range(tp):
        ys = np.ascontiguousarray(yf[:, r * h_r:(r + 1) * h_r])
        ws = np.ascontiguousarray(w_o[:, r * h_r * d:(r + 1) * h_r * d])
        parts.append(oracle.o_wo_partial(ys, ws))
        tt.tp_o_wo_partial(dev_bf16(ys).view(M, -1), heads, padded, qkv, ff, tp, r, dev_bf16(ws), out, accumulate=r > 0)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), oracle.rank_ordered_sum(parts), tol=1e-4, what="rank-ordered o_wo sum")


def test_chain_qwi_swiglu_o_wo():
    """q_wi -> SwiGLU into y_fused next to a synthetic attention output -> o_wo partial."""
    M, E, heads, padded, qkv, ff, tp, rank = 256, 512, 8, 0, 64, 1024, 2, 0  # fph 128
    h_r, fph, qph = oracle.qwi_dims(heads, padded, qkv, ff, tp)
    x = synth.bf16_normal((M, E), 1.0, 64, 0)
    w = synth.bf16_normal((h_r * qph, E), 0.02, 64, 1)
    w_o = synth.bf16_normal((E, h_r * (qkv + fph)), 0.02, 64, 2)
    y_att = synth.bf16_normal((M, h_r, qkv), 1.0, 64, 3)
    _, y_mlp = oracle.qwi_swiglu(x, w, heads, padded, qkv, ff, tp, rank)
    ref = oracle.o_wo_partial(oracle.fuse_heads(y_att, y_mlp), w_o)
    yf = torch.empty((M, h_r, qkv + fph), dtype=torch.bfloat16, device="cuda")
    yf[:, :, :qkv] = dev_bf16(y_att)
    tt.tp_qwi_swiglu(dev_bf16(x), heads, padded, qkv, ff, tp, rank, dev_bf16(w), yf)
    out = tt.tp_o_wo_partial(yf.view(M, -1), heads, padded, qkv, ff, tp, rank, dev_bf16(w_o))
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, what="q_wi -> SwiGLU -> o_wo")


def test_full_size_sampled_rows():
    """8192 tokens, E 8192, 64 heads of 128, d_ff 32768, tp 8 rank 0: all outputs computed on
    the GPU, sampled rows checked against the oracle."""
    M, E, heads, padded, qkv, ff, tp, rank = 8192, 8192, 64, 0, 128, 32768, 8, 0
    h_r, fph, qph = oracle.qwi_dims(heads, padded, qkv, ff, tp)
    x = synth.bf16_normal((M, E), 1.0, 65, 0)
    w = synth.bf16_normal((h_r * qph, E), 0.02, 65, 1)
    w_o = synth.bf16_normal((E, h_r * (qkv + fph)), 0.02, 65, 2)
    xd, wd, wod = dev_bf16(x), dev_bf16(w), dev_bf16(w_o)
    yf = torch.zeros((M, h_r, qkv + fph), dtype=torch.bfloat16, device="cuda")
    q = torch.empty((M, h_r, qkv), dtype=torch.bfloat16, device="cuda")
    tt.tp_qwi_swiglu(xd, heads, padded, qkv, ff, tp, rank, wd, yf, q=q)
    out = tt.tp_o_wo_partial(yf.view(M, -1), heads, padded, qkv, ff, tp, rank, wod)
    torch.cuda.synchronize()
    rows = np.random.default_rng(66).choice(M, 24, replace=False)
    rows[:2] = [0, M - 1]
    q_ref, y_ref = oracle.qwi_swiglu(x[rows], w, heads, padded, qkv, ff, tp, rank)
    qb, yb = host_bits(q)[rows], host_bits(yf)[rows]
    assert_close(qb, q_ref, what="q (sampled rows)")
    assert_close(yb[:, :, qkv:], y_ref, what="swiglu (sampled rows)", straddle=5e-3, ulps=2)
    assert not np.any(oracle.bf16_to_f64(yb[:, :, :qkv])), "attention slots were written"
    # the o_wo partial from the GPU's own y_fused rows: the projection alone
    ref = oracle.o_wo_partial(yb, w_o)
    assert_close(out.cpu().numpy()[rows], ref, tol=1e-4, what="o_wo (sampled rows)")
    assert TOL == 2e-2
