"""Pins of the oracle's RMSNorm prologue: special cases, torch dtype semantics, brute force."""
import math
import struct

import numpy as np
import pytest
import torch

import oracle
import synth


def _f32(v):
    return struct.unpack("f", struct.pack("f", v))[0]


def _torch_rmsnorm(x_bits, scale_bits, eps=1e-6):
    """The same steps written with torch CPU dtype semantics (float32 statistics, bf16 casts).

    Statistics are taken in float64 and rounded to float32 once, as the oracle's
    reading states (the page's float32 mean differs only in summation rounding).
    """
    x = torch.from_numpy(x_bits.view(np.int16).copy()).view(torch.bfloat16)
    xf = x.to(torch.float32)
    ms = (x.to(torch.float64) ** 2).mean(dim=-1, keepdim=True)
    r = torch.rsqrt(ms + eps).to(torch.float32)
    n = (xf * r).to(torch.bfloat16)
    if scale_bits is None:
        return n.view(torch.int16).numpy().view(np.uint16)
    s = torch.from_numpy(scale_bits.view(np.int16).copy()).view(torch.bfloat16)
    t = s + 1.0  # bf16 + python float stays bf16 (computed in float32, rounded once)
    y = n * t    # bf16 * bf16 -> bf16
    return y.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("scaled", [False, True])
def test_rmsnorm_matches_torch_dtype_semantics(scaled):
    g = np.random.default_rng(21)
    x = synth.bf16_from_float(g.standard_normal((64, 512)) * 1.7)
    s = synth.bf16_from_float(g.standard_normal(512) * 0.1) if scaled else None
    y, _ = oracle.rmsnorm(x, s)
    ref = _torch_rmsnorm(x, s)
    # the only freedom is the last float32 ulp of r (float64 vs torch's rsqrt); allow
    # a handful of 1-ulp bf16 differences and nothing larger
    diff = np.abs(y.astype(np.int32) - ref.astype(np.int32))
    assert diff.max() <= 1
    assert np.count_nonzero(diff) <= 0.002 * diff.size


def test_rmsnorm_unit_rows():
    """Rows of +-1: mean square 1, r = f32(1/sqrt(1 + eps)), n = bf16(+-r)."""
    K = 256
    g = np.random.default_rng(3)
    x = synth.bf16_from_float(np.where(g.random((4, K)) < 0.5, -1.0, 1.0))
    y, r = oracle.rmsnorm(x)
    r_want = _f32(1.0 / math.sqrt(1.0 + 1e-6))
    assert np.all(r == np.float32(r_want))
    pos = int(torch.tensor([r_want]).to(torch.bfloat16).view(torch.int16).item()) & 0xFFFF
    assert np.all(y == np.where(oracle.bf16_to_f64(x) > 0, pos, pos | 0x8000))


def test_rmsnorm_zero_row_and_k1():
    x = np.zeros((1, 64), dtype=np.uint16)
    y, r = oracle.rmsnorm(x)
    assert r[0] == np.float32(1000.0) and np.all(y == 0)
    # K = 1: r = 1/sqrt(x^2 + eps), n = bf16(x r) which is ~sign(x)
    x1 = synth.bf16_from_float(np.array([[3.0], [-0.25]]))
    y1, r1 = oracle.rmsnorm(x1)
    assert r1[0] == np.float32(1.0 / math.sqrt(9.0 + 1e-6))
    assert r1[1] == np.float32(1.0 / math.sqrt(0.0625 + 1e-6))
    assert abs(oracle.bf16_to_f64(y1[0, 0]) - 1.0) < 2 ** -7
    assert abs(oracle.bf16_to_f64(y1[1, 0]) + 1.0) < 2 ** -7


def test_rmsnorm_zero_scale_equals_unscaled():
    g = np.random.default_rng(8)
    x = synth.bf16_from_float(g.standard_normal((8, 96)))
    zero = np.zeros(96, dtype=np.uint16)
    assert np.array_equal(oracle.rmsnorm(x, zero)[0], oracle.rmsnorm(x)[0])


def test_scale_plus_one_is_rounded_to_bf16_first():
    """t = bf16(1 + s): a scale whose 1 + s is not a bf16 value shows the rounding."""
    s = synth.bf16_from_float(np.array([2.0 ** -9 * 1.5]))   # 1 + s needs 10 significant bits
    x = synth.bf16_from_float(np.array([[1.0]]))
    y, r = oracle.rmsnorm(x, s)
    n = oracle.bf16_round(np.array([_f32(1.0 * float(r[0]))], dtype=np.float32))
    t_bf16 = 1.0 + 2.0 ** -8  # bf16(1 + 1.5 * 2^-9) ties to even -> 1 + 2^-8
    want = oracle.bf16_round(np.array([_f32(oracle.bf16_to_f64(n[0]) * t_bf16)], dtype=np.float32))
    assert y[0, 0] == want[0]


def test_rmsnorm_brute_force():
    """Python-float statistics and struct float32 rounding, torch bf16 rounding, 32K elements exact."""
    g = np.random.default_rng(12)
    M, K = 64, 512
    x = synth.bf16_from_float(g.standard_normal((M, K)))
    s = synth.bf16_from_float(g.standard_normal(K) * 0.1)
    y, r = oracle.rmsnorm(x, s)
    sv = [float(v) for v in oracle.bf16_to_f64(s)]
    t = torch.tensor([_f32(1.0 + v) for v in sv]).to(torch.bfloat16).to(torch.float64)
    for m in range(M):
        vals = [float(v) for v in oracle.bf16_to_f64(x[m])]
        ms = math.fsum(v * v for v in vals) / K
        rr = _f32(1.0 / math.sqrt(ms + 1e-6))
        assert r[m] == np.float32(rr)
        n = torch.tensor([_f32(v * rr) for v in vals]).to(torch.bfloat16).to(torch.float64)
        want = (n * t).to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(y[m], want)


def test_rmsnorm_column_linear_composes():
    g = np.random.default_rng(13)
    x = synth.bf16_from_float(g.standard_normal((4, 64)))
    s = synth.bf16_from_float(g.standard_normal(64) * 0.1)
    w = synth.bf16_from_float(g.standard_normal((12, 64)) * 0.1)
    y, xn = oracle.rmsnorm_column_linear(x, s, w[:6], None, [12], 2, 0)
    assert np.array_equal(xn, oracle.rmsnorm(x, s)[0])
    assert np.array_equal(y, oracle.column_linear(xn, w[:6], None, [12], 2, 0))
