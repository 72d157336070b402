"""Pins of the oracle's fp8 prefill pieces (E4M3 encoder, per-row activation quantiser, fp8
column linear) against torch's float8 cast, brute force over the code table, closed forms
and integer arithmetic."""
import numpy as np
import pytest
import torch

import oracle
import synth


def _finite_codes():
    return np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def test_encode_matches_torch_float8_cast_in_range():
    g = np.random.default_rng(11)
    v = np.concatenate([g.standard_normal(20000) * 40, g.standard_normal(20000) * 1e-2,
                        g.uniform(-447.9, 447.9, 20000)]).astype(np.float32)
    v = np.concatenate([v, np.array([0.0, -0.0, -1e-9, 1e-9], np.float32)])
    ours = oracle.e4m3_encode(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref), v[ours != ref][:5]  # signed zero included


def test_encode_is_nearest_by_brute_force():
    g = np.random.default_rng(12)
    v = (g.standard_normal(3000) * g.choice([1e-3, 1e-1, 1, 30, 300], 3000)).astype(np.float32)
    v = np.clip(v, -448, 448)
    codes = _finite_codes()
    vals = oracle.e4m3_to_f64(codes)
    got = oracle.e4m3_to_f64(oracle.e4m3_encode(v))
    best = np.min(np.abs(vals[None, :] - v.astype(np.float64)[:, None]), axis=1)
    assert np.array_equal(np.abs(got - v), best)


def test_encode_ties_go_to_the_even_code_and_large_values_saturate():
    vals = oracle.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)  # every midpoint is a float32
    assert np.array_equal(mids.astype(np.float64), (vals[:-1] + vals[1:]) / 2)
    codes = oracle.e4m3_encode(mids)
    lo = np.arange(0x7E, dtype=np.uint8)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(codes, expect)
    assert np.array_equal(oracle.e4m3_encode(-mids), expect | 0x80)
    big = np.array([448, 449, 464, 480, 1e6, -500], np.float32)
    assert np.array_equal(oracle.e4m3_encode(big), np.array([0x7E] * 5 + [0xFE], np.uint8))


def test_quantize_rows_closed_forms():
    x = np.zeros((4, 64), np.uint16)
    x[1, 5] = synth.bf16_from_float(np.array([-3.0]))[0]  # one-hot row: scale 3/448, code -448
    x[2] = synth.bf16_integers((1, 64), -7, 7, 3)[0]
    x[3] = synth.bf16_from_float(np.full(64, 2.0 ** -20))
    q, s = oracle.quantize_rows_e4m3(x)
    assert s[0] == 1.0 and not q[0].any()
    assert s[1] == np.float32(3.0) / np.float32(448) and q[1, 5] == 0xFE and (q[1, np.arange(64) != 5] == 0).all()
    amax = np.abs(synth_vals := oracle.bf16_to_f64(x[2])).max()
    assert s[2] == np.float32(amax) / np.float32(448)
    # the quantised row reproduces x within half an E4M3 step (3 mantissa bits: 2^-4 relative)
    rec = oracle.e4m3_to_f64(q[2]) * s[2]
    assert np.all(np.abs(rec - synth_vals) <= 2.0 ** -4 * np.abs(synth_vals) + 1e-12)
    assert (q[3] == 0x7E).all()  # a constant row: every element is the row maximum


def test_quantize_rows_error_bound_on_gaussian_rows():
    x = synth.bf16_normal((64, 512), 1.0, 901, 0)
    q, s = oracle.quantize_rows_e4m3(x)
    xf = oracle.bf16_to_f64(x)
    rec = oracle.e4m3_to_f64(q) * s[:, None].astype(np.float64)
    # normal E4M3 values: half a step relative; subnormal quotients: half of 2^-9 absolute
    bound = np.maximum(2.0 ** -4 * np.abs(xf), 2.0 ** -10 * s[:, None]) * (1 + 1e-6)
    assert np.all(np.abs(rec - xf) <= bound)
    assert np.all(np.abs(oracle.e4m3_to_f64(q)).max(axis=1) == 448)


def test_fp8_linear_exact_on_integer_codes_and_power_of_two_scales():
    g = np.random.default_rng(5)
    ints = np.array([-4, -3, -2, -1, 0, 1, 2, 3, 4], np.float32)
    M, N, K = 7, 12, 64
    xv = g.choice(ints, (M, K)); wv = g.choice(ints, (N, K))
    xq, wq = oracle.e4m3_encode(xv), oracle.e4m3_encode(wv)
    assert np.array_equal(oracle.e4m3_to_f64(xq), xv) and np.array_equal(oracle.e4m3_to_f64(wq), wv)
    xs = (2.0 ** g.integers(-3, 4, M)).astype(np.float32)
    ws = (2.0 ** g.integers(-3, 4, N)).astype(np.float32)
    y = oracle.column_linear_fp8(xq, xs, wq, ws, None, [N], 1, 0, out_dtype=oracle.OUT_F32)
    ref = (xv.astype(np.int64) @ wv.astype(np.int64).T).astype(np.float64) * xs[:, None] * ws[None, :]
    assert np.array_equal(y.astype(np.float64), ref)


def test_fp8_linear_brute_force_with_bias_gelu_and_shards():
    g = np.random.default_rng(6)
    M, K = 3, 32
    sizes = [10, 6]
    tp = 2
    wq_full = oracle.e4m3_encode((g.standard_normal((16, K)) * 3).astype(np.float32))
    ws_full = g.uniform(0.01, 0.1, 16).astype(np.float32)
    b_full = synth.bf16_normal((16,), 0.5, 902, 2)
    xq = oracle.e4m3_encode((g.standard_normal((M, K)) * 20).astype(np.float32))
    xs = g.uniform(0.01, 0.1, M).astype(np.float32)
    parts = []
    for r in range(tp):
        rows = oracle.shard_rows(sizes, tp, r)
        y = oracle.column_linear_fp8(xq, xs, wq_full[rows], ws_full[rows], b_full[rows], sizes, tp, r,
                                     act=oracle.ACT_GELU)
        # brute force in Python for this shard
        for m in range(M):
            for j, n in enumerate(rows):
                acc = sum(oracle.e4m3_to_f64(xq[m, k]) * oracle.e4m3_to_f64(wq_full[n, k]) for k in range(K))
                a = np.float32(xs[m] * np.float64(ws_full[n]) * acc + oracle.bf16_to_f64(b_full[n]))
                a = np.float32(oracle.gelu_erf(np.array([a], np.float32))[0])
                assert y[m, j] == oracle.bf16_round(np.array([a], np.float32))[0]
        out, mask = oracle.column_linear_fp8(xq, xs, wq_full[rows], ws_full[rows], b_full[rows], sizes, tp, r,
                                             act=oracle.ACT_GELU, layout=oracle.LAYOUT_LOGICAL)
        parts.append((out, mask))
    full = oracle.column_linear_fp8(xq, xs, wq_full, ws_full, b_full, [16], 1, 0, act=oracle.ACT_GELU)
    # LOGICAL shards of both ranks cover the unsharded output exactly once (columns by sub-param)
    cover = parts[0][1].astype(int) + parts[1][1].astype(int)
    assert (cover == 1).all()
    assembled = np.where(parts[0][1][None, :], parts[0][0], parts[1][0])
    assert np.array_equal(assembled, full)


def test_channel_quantised_weights_decode_within_half_a_step():
    w = synth.bf16_normal((48, 256), 0.02, 903, 1)
    q, s = synth.quantize_e4m3_channels(w)
    assert s.shape == (48,)
    wf = oracle.bf16_to_f64(w)
    rec = oracle.e4m3_to_f64(q) * s[:, None].astype(np.float64)
    bound = np.maximum(2.0 ** -4 * np.abs(wf), 2.0 ** -10 * s[:, None]) * (1 + 1e-6)
    assert np.all(np.abs(rec - wf) <= bound)
    # the generator's encoder and the oracle's agree on the stored codes
    assert np.array_equal(q, oracle.e4m3_encode((wf / s[:, None]).astype(np.float32)))


def test_straddle_rule_accepts_only_roundings_within_the_accumulation_bound():
    """The GPU tests' acceptance rule for bf16 outputs (helpers.check_bf16): an output one unit
    away from the oracle's is accepted only where the exact sum lies within the accumulation
    bound of the bf16 rounding boundary between the two."""
    import helpers
    def b(v):
        return int(oracle.bf16_round(np.float32(v))[0])
    # row 0: 1 + 2^-8 + 2^-20, a hair above the midpoint of 1.0 and 1.0078125 -> the oracle rounds up
    # row 1: 1.25: far from any boundary
    x = np.array([[b(1), b(1), b(2.0 ** -20)], [b(1.25), 0, 0]], dtype=np.uint16)
    w = np.array([[b(1), b(2.0 ** -8), b(1)], [b(1), b(1), b(1)]], dtype=np.uint16)
    v = oracle.linear_sums(x, w)
    ref = oracle.column_linear(x, w, None, [2], 1, 0)
    assert v[0, 0] == 1 + 2.0 ** -8 + 2.0 ** -20 and oracle.bf16_to_f64(ref[0, 0]) == 1.0078125
    sums = helpers.AbsSums.bf16(x, w)
    assert helpers.check_bf16(ref, ref, v, sums) == 0
    got = ref.copy()
    got[0, 0] -= 1                                 # the other side of the boundary: a straddle
    assert helpers.check_bf16(got, ref, v, sums) == 1
    far = ref.copy()
    far[1, 0] += 1                                 # one unit off, nowhere near a boundary
    with pytest.raises(AssertionError, match="not rounding straddles"):
        helpers.check_bf16(far, ref, v, sums)
    with pytest.raises(AssertionError, match="not rounding straddles"):  # the straddle window is narrow
        helpers.check_bf16(got, ref, v, sums, c=2.0 ** -30)
    big = ref.copy()
    big[1, 1] ^= 0x4000
    with pytest.raises(AssertionError):
        helpers.check_bf16(big, ref, v, sums)


def test_f32_rule_holds_each_output_to_the_accumulation_bound():
    import helpers
    g = np.random.default_rng(3)
    x = synth.bf16_from_float(g.standard_normal((8, 512)))
    w = synth.bf16_from_float(g.standard_normal((16, 512)) * 0.02)
    v = oracle.linear_sums(x, w)
    sums = helpers.AbsSums.bf16(x, w).block(0, 8)
    helpers.check_f32(oracle.f32(v), v, sums)
    off = oracle.f32(v).astype(np.float64)
    off[3, 4] += 4e-3 * sums[3, 4] * 2.0 ** -10
    with pytest.raises(AssertionError, match="beyond the accumulation bound"):
        helpers.check_f32(off, v, sums)


def test_swiglu_rule_accepts_only_admissible_gate_value_roundings():
    """helpers.check_swiglu: the GPU's SwiGLU output must be the rounding of swish(g) * u for bf16
    g, u within the accumulation bound of the exact sums; a value that moved although neither sum
    is near a bf16 boundary is rejected, one whose value sum sits on a boundary is accepted."""
    import helpers

    def b(v):
        return int(oracle.bf16_round(np.float32(v))[0])
    # row 0: gate 1, value 1 + 2^-8 + 2^-20 (a hair above the midpoint of 1 and 1.0078125);
    # row 1: gate 2, value 1.25, far from any boundary
    x = np.array([[b(1), b(1), b(2.0 ** -20)], [b(1), 0, 0]], dtype=np.uint16)
    wg = np.array([[b(1), 0, 0], [b(2), 0, 0]], dtype=np.uint16)[[0, 0]]
    wu = np.array([[b(1), b(2.0 ** -8), b(1)]], dtype=np.uint16)
    # one head, qkv 0: gate rows [g], value rows [u]; columns: the two rows of x against one gate/value
    gate = oracle.linear_sums(x, wg[:1])
    value = oracle.linear_sums(x, wu)
    gb = oracle.bf16_round(oracle.f32(gate))
    ub = oracle.bf16_round(oracle.f32(value))
    ref = oracle.bf16_round(oracle.f32(oracle.swish(oracle.bf16_to_f64(gb)) * oracle.bf16_to_f64(ub)))
    gs, us = helpers.AbsSums.bf16(x, wg[:1]), helpers.AbsSums.bf16(x, wu)
    assert helpers.check_swiglu(ref, ref, gate, value, gs, us) == 0
    # row 0 with the value rounded down instead (1.0): an admissible other rounding
    alt = ref.copy()
    alt[0, 0] = oracle.bf16_round(oracle.f32(oracle.swish(oracle.bf16_to_f64(gb[0, 0])) * 1.0))[0]
    assert alt[0, 0] != ref[0, 0]
    assert helpers.check_swiglu(alt, ref, gate, value, gs, us) == 1
    # row 1 one unit off: its sums are far from any boundary
    bad = ref.copy()
    bad[1, 0] += 1
    with pytest.raises(AssertionError, match="not roundings"):
        helpers.check_swiglu(bad, ref, gate, value, gs, us)
