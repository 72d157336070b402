"""Pins of the oracle's fused q_wi + SwiGLU projection and o_wo partial ([palm] q_wi, SwiGLU, o_wo).

Each pin comes from outside the oracle's own formulas: scipy's logistic function, closed forms
of the Swish, brute-force Python loops that index each head's rows one by one, and the
invariants of the head split (the ranks' heads concatenated give the unsharded result, the
ranks' o_wo partials sum to the unsharded contraction).
"""
import math

import numpy as np
import pytest
from scipy.special import expit

import oracle
import synth


def _bits(a):
    return oracle.bf16_round(np.asarray(a, dtype=np.float32))


def _bit1(v) -> np.uint16:
    """bf16 bits of one float32 value."""
    return _bits(np.array([v], dtype=np.float32))[0]


def test_swish_matches_logistic_times_input():
    v = np.linspace(-40.0, 40.0, 4001)
    np.testing.assert_allclose(oracle.swish(v), v * expit(v), rtol=1e-14, atol=1e-300)


def test_swish_closed_forms_and_limits():
    # sigmoid(ln 3) = 3/4, sigmoid(0) = 1/2
    assert oracle.swish(math.log(3.0)) == pytest.approx(0.75 * math.log(3.0), rel=1e-15)
    assert oracle.swish(0.0) == 0.0
    assert oracle.swish(1e4) == 1e4
    big_neg = oracle.swish(-1e4)
    assert big_neg == 0.0 and math.copysign(1.0, big_neg) == -1.0
    # v sigmoid(v) - (-v) sigmoid(-v) = v: catches a sign error in the exponent
    v = np.array([-7.5, -1.25, 0.3, 2.0, 9.0])
    np.testing.assert_allclose(oracle.swish(v) - oracle.swish(-v), v, rtol=1e-14)


def test_dims_follow_the_real_heads():
    # ff spread over heads - padded_heads, floor division; padded heads carry the same width
    assert oracle.qwi_dims(6, 1, 32, 200, 2) == (3, 40, 112)
    assert oracle.qwi_dims(5, 1, 4, 10, 5) == (1, 2, 8)
    assert oracle.qwi_dims(64, 0, 128, 32768, 8) == (8, 512, 1152)
    with pytest.raises(ValueError):
        oracle.qwi_dims(6, 0, 32, 200, 4)  # heads do not split over 4 ranks
    with pytest.raises(ValueError):
        oracle.qwi_dims(6, 6, 32, 200, 2)  # no real head
    with pytest.raises(ValueError):
        oracle.qwi_dims(6, 1, 32, 4, 2)  # ff < real heads


def _brute_qwi(x_bits, w_bits, h_r, qkv, fph):
    """Pure-Python loops: each output from its own rows, Swish from math.exp."""
    x = oracle.bf16_to_f64(x_bits)
    w = oracle.bf16_to_f64(w_bits)
    M, E = x.shape
    qph = qkv + 2 * fph

    def dot(m, row):
        s = 0.0
        for e in range(E):
            s += x[m, e] * w[row, e]
        return s

    def bf(v):
        return float(oracle.bf16_to_f64(_bit1(v)))

    q = np.zeros((M, h_r, qkv), dtype=np.uint16)
    y = np.zeros((M, h_r, fph), dtype=np.uint16)
    for m in range(M):
        for h in range(h_r):
            base = h * qph
            for d in range(qkv):
                q[m, h, d] = _bit1(dot(m, base + d))
            for j in range(fph):
                g = bf(dot(m, base + qkv + j))
                u = bf(dot(m, base + qkv + fph + j))
                y[m, h, j] = _bit1(g / (1.0 + math.exp(-g)) * u)
    return q, y


def test_qwi_swiglu_brute_force_small():
    heads, padded, qkv, ff, tp = 4, 1, 3, 7, 2  # fph = 7 // 3 = 2
    h_r, fph, qph = oracle.qwi_dims(heads, padded, qkv, ff, tp)
    x = synth.bf16_normal((5, 12), 1.0, 40, 0)
    w = synth.bf16_normal((h_r * qph, 12), 0.5, 40, 1)
    q, y = oracle.qwi_swiglu(x, w, heads, padded, qkv, ff, tp, 1)
    qb, yb = _brute_qwi(x, w, h_r, qkv, fph)
    assert q.shape == (5, h_r, qkv) and y.shape == (5, h_r, fph)
    np.testing.assert_array_equal(q, qb)
    np.testing.assert_array_equal(y, yb)


def test_qwi_swiglu_gate_and_value_are_not_interchangeable():
    # one head, one MLP column: wi0 = 2, wi1 = -3 -> swish(2) * -3, not swish(-3) * 2
    x = _bits(np.array([[1.0, 1.0]], dtype=np.float32))
    w = _bits(np.array([[0.0, 0.0], [1.0, 1.0], [-1.0, -2.0]], dtype=np.float32))  # q, wi0, wi1 rows
    q, y = oracle.qwi_swiglu(x, w, 1, 0, 1, 1, 1, 0)
    assert y[0, 0, 0] == _bit1(2.0 / (1.0 + math.exp(-2.0)) * -3.0)
    assert oracle.bf16_to_f64(q[0, 0, 0]) == 0.0


def test_head_shards_concatenate_to_the_unsharded_result():
    heads, padded, qkv, ff = 6, 0, 4, 30  # fph 5
    h_all, fph, qph = oracle.qwi_dims(heads, padded, qkv, ff, 1)
    x = synth.bf16_normal((7, 16), 1.0, 41, 0)
    w_full = synth.bf16_normal((h_all * qph, 16), 0.3, 41, 1)
    q_full, y_full = oracle.qwi_swiglu(x, w_full, heads, padded, qkv, ff, 1, 0)
    tp = 3
    h_r = heads // tp
    qs, ys = [], []
    for r in range(tp):
        w_r = w_full[r * h_r * qph:(r + 1) * h_r * qph]
        q_r, y_r = oracle.qwi_swiglu(x, w_r, heads, padded, qkv, ff, tp, r)
        qs.append(q_r)
        ys.append(y_r)
    np.testing.assert_array_equal(np.concatenate(qs, axis=1), q_full)
    np.testing.assert_array_equal(np.concatenate(ys, axis=1), y_full)


def test_padded_heads_with_zero_weights_give_zero_outputs():
    heads, padded, qkv, ff, tp = 4, 2, 2, 6, 2  # fph 3; rank 1 holds the two padded heads
    h_r, fph, qph = oracle.qwi_dims(heads, padded, qkv, ff, tp)
    x = synth.bf16_normal((3, 8), 1.0, 42, 0)
    w = np.zeros((h_r * qph, 8), dtype=np.uint16)
    q, y = oracle.qwi_swiglu(x, w, heads, padded, qkv, ff, tp, 1)
    assert not np.any(oracle.bf16_to_f64(q)) and not np.any(oracle.bf16_to_f64(y))


def test_fuse_heads_places_attention_then_mlp_per_head():
    att = np.arange(2 * 3 * 2, dtype=np.uint16).reshape(2, 3, 2)
    mlp = (100 + np.arange(2 * 3 * 4, dtype=np.uint16)).reshape(2, 3, 4)
    f = oracle.fuse_heads(att, mlp)
    assert f.shape == (2, 3, 6)
    for m in range(2):
        for h in range(3):
            assert list(f[m, h]) == list(att[m, h]) + list(mlp[m, h])


def test_o_wo_partials_sum_to_the_unsharded_contraction():
    heads, qkv, fph, E, M, tp = 4, 3, 5, 6, 4, 2
    d = qkv + fph
    yf = synth.bf16_normal((M, heads, d), 1.0, 43, 0)
    w_o = synth.bf16_normal((E, heads * d), 0.5, 43, 1)  # column h * d + t is head h, position t
    h_r = heads // tp
    parts = [oracle.o_wo_partial(yf[:, r * h_r:(r + 1) * h_r], w_o[:, r * h_r * d:(r + 1) * h_r * d])
             for r in range(tp)]
    # brute force over heads and positions
    yv, wv = oracle.bf16_to_f64(yf), oracle.bf16_to_f64(w_o)
    want = np.zeros((M, E))
    for m in range(M):
        for e in range(E):
            s = 0.0
            for h in range(heads):
                for t in range(d):
                    s += yv[m, h, t] * wv[e, h * d + t]
            want[m, e] = s
    total = parts[0].astype(np.float64) + parts[1].astype(np.float64)
    np.testing.assert_allclose(total, want, rtol=1e-6, atol=1e-6 * np.abs(want).max())
    # each part is the exact contraction over its heads, rounded once to float32
    for r in range(tp):
        s = np.zeros((M, E))
        for h in range(r * h_r, (r + 1) * h_r):
            s += yv[:, h, :] @ wv[:, h * d:(h + 1) * d].T
        np.testing.assert_array_equal(parts[r], s.astype(np.float32))
