"""Pins of the oracle's number codecs against library routines and the formats' definitions."""
import numpy as np
import pytest
import torch

import oracle
import synth


def _torch_bf16_bits(v32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_round_matches_torch_on_random_patterns():
    g = np.random.default_rng(1)
    u = g.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    v = u.view(np.float32)
    v = v[~np.isnan(v)]
    assert np.array_equal(oracle.bf16_round(v), _torch_bf16_bits(v))


@pytest.mark.parametrize("pattern,expected", [
    (0x3F800000, 0x3F80),  # 1.0
    (0x3F808000, 0x3F80),  # exact tie, kept pattern even -> down
    (0x3F818000, 0x3F82),  # exact tie, kept pattern odd -> up
    (0x3F808001, 0x3F81),  # above the tie -> up
    (0x3F807FFF, 0x3F80),  # below the tie -> down
    (0x7F7F0000, 0x7F7F),  # largest finite bf16
    (0x7F7FFFFF, 0x7F80),  # rounds past the largest finite -> +inf
    (0x00010000, 0x0001),  # subnormal, exact
    (0x80000000, 0x8000),  # -0
    (0xFF800000, 0xFF80),  # -inf
])
def test_bf16_round_edge_patterns(pattern, expected):
    v = np.array([pattern], dtype=np.uint32).view(np.float32)
    assert int(oracle.bf16_round(v)[0]) == expected


def test_bf16_decode_is_exact_widening():
    bits = np.arange(0, 2 ** 16, dtype=np.uint32).astype(np.uint16)
    d = oracle.bf16_to_f64(bits)
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    fin = ~np.isnan(t)
    assert np.array_equal(d[fin], t[fin])
    assert np.array_equal(np.isnan(d), np.isnan(t))


def test_e4m3_table_matches_torch_float8_e4m3fn():
    codes = np.arange(256, dtype=np.uint8)
    t = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    o = oracle.e4m3_table()
    assert np.array_equal(np.isnan(o), np.isnan(t))
    fin = ~np.isnan(o)
    assert np.array_equal(o[fin], t[fin])


def test_e4m3_table_known_codes():
    t = oracle.e4m3_table()
    assert t[0x00] == 0.0 and t[0x80] == 0.0
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0          # largest finite
    assert t[0x01] == 2.0 ** -9                            # smallest subnormal
    assert t[0x08] == 2.0 ** -6                            # smallest normal
    assert t[0x38] == 1.0                                  # e = 7, m = 0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert int(np.sum(np.isnan(t))) == 2                   # no infinities, two NaNs
    # every finite E4M3 value is exactly a bf16 value (needed for exact dequantisation)
    fin = t[~np.isnan(t)].astype(np.float32)
    assert np.array_equal(oracle.bf16_to_f64(oracle.bf16_round(fin)), fin.astype(np.float64))


def test_synth_quantiser_is_nearest_code():
    """The stored E4M3 codes are the nearest representable value of w/scale (ties even)."""
    w = synth.bf16_normal((64, 256), 0.02, 77, 1)
    q, s = synth.quantize_e4m3_blocks(w)
    assert q.dtype == np.uint8 and s.shape == (64, 2)
    assert not np.any((q & 0x7F) == 0x7F)
    t = oracle.e4m3_table()
    wf = oracle.bf16_to_f64(w).reshape(64, 2, 128)
    target = (wf.astype(np.float32) / s[:, :, None]).astype(np.float64)
    got = t[q.reshape(64, 2, 128)]
    fin = t[~np.isnan(t)]
    # distance to the chosen code is minimal over all codes
    best = np.min(np.abs(target[..., None] - fin[None, None, None, :]), axis=-1)
    assert np.array_equal(np.abs(target - got), best)
    # per block, the largest magnitude maps to 448 exactly
    assert np.all(np.max(np.abs(got), axis=2) == 448.0)


def test_synth_chunked_draw_equals_single_draw():
    a = synth.bf16_normal((1000, 64), 1.0, 5, 0, chunk_rows=128)
    b = synth.bf16_normal((1000, 64), 1.0, 5, 0, chunk_rows=10_000)
    assert np.array_equal(a, b)
    c = synth._first_rows_normal(300, 64, 1.0, 5, 0)
    assert np.array_equal(a[:300], c)


def test_synth_bf16_matches_torch_rounding():
    g = np.random.default_rng(3)
    v = g.standard_normal(10000).astype(np.float32)
    assert np.array_equal(synth.bf16_from_float(v), _torch_bf16_bits(v))
