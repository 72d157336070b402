"""Pins of the oracle's vocab-sharded LM head and per-shard argmax."""
import numpy as np
import pytest

import oracle
import synth


def test_chunked_equals_unchunked_bitwise():
    g = np.random.default_rng(31)
    x = synth.bf16_from_float(g.standard_normal((8, 256)))
    w = synth.bf16_from_float(g.standard_normal((103, 256)) * 0.02)
    full = oracle.lm_head_logits(x, w)
    for c in (1, 7, 50, 103, 500):
        assert np.array_equal(oracle.lm_head_logits(x, w, max_rows_per_chunk=c), full)
    q, s = synth.quantize_e4m3_blocks(w)
    f8 = oracle.lm_head_logits(x, w_fp8=q, w_scale=s)
    for c in (13, 64):
        assert np.array_equal(oracle.lm_head_logits(x, w_fp8=q, w_scale=s, max_rows_per_chunk=c), f8)


def test_bf16_logits_are_textbook_matmul():
    g = np.random.default_rng(32)
    x = synth.bf16_from_float(g.standard_normal((4, 128)))
    w = synth.bf16_from_float(g.standard_normal((9, 128)))
    got = oracle.lm_head_logits(x, w)
    xs = oracle.bf16_to_f64(x)
    ws = oracle.bf16_to_f64(w)
    brute = np.array([[sum(xs[b, k] * ws[v, k] for k in range(128)) for v in range(9)] for b in range(4)])
    assert np.max(np.abs(got - brute.astype(np.float32))) <= 1e-6 * np.max(np.abs(brute))


def test_fp8_exact_with_integer_codes_and_power_of_two_scales():
    """Integer x, integer E4M3 values and power-of-two scales: logits are exact integers / powers of 2."""
    g = np.random.default_rng(33)
    B, V, K = 3, 10, 256
    x = synth.bf16_integers((B, K), -4, 4, 40)
    ints = g.integers(-8, 9, size=(V, K))
    # E4M3 codes of small integers from the format: 1 -> 0x38, 2 -> 0x40, 3 -> 0x44, ...
    table = oracle.e4m3_table()
    code_of = {float(table[c]): c for c in range(256) if not np.isnan(table[c]) and c != 0x80}
    q = np.vectorize(lambda v: code_of[float(v)])(ints).astype(np.uint8)
    s = (2.0 ** g.integers(-3, 4, size=(V, K // 128))).astype(np.float32)
    got = oracle.lm_head_logits(x, w_fp8=q, w_scale=s, max_rows_per_chunk=4)
    xi = oracle.bf16_to_f64(x)
    want = np.zeros((B, V))
    for blk in range(K // 128):
        ks = slice(blk * 128, blk * 128 + 128)
        want += (xi[:, ks] @ ints[:, ks].T) * s[:, blk][None, :]
    assert np.array_equal(got, want.astype(np.float32))


def test_vocab_shards_concatenate_to_full_vocab():
    """Each shard holds the correct logits for its vocab rows (no partial sums)."""
    g = np.random.default_rng(34)
    vocab, tp, K = 203, 8, 128
    x = synth.bf16_from_float(g.standard_normal((5, K)))
    w = synth.bf16_from_float(g.standard_normal((vocab, K)) * 0.05)
    full = oracle.lm_head_logits(x, w)
    parts, idx_max = [], []
    for r in range(tp):
        rows, off = oracle.vocab_shard(vocab, tp, r)
        lg = oracle.lm_head_logits(x, w[off:off + rows], max_rows_per_chunk=6)
        parts.append(lg)
        i, m = oracle.shard_argmax(lg)
        idx_max.append((i, m, off))
    assert np.array_equal(np.concatenate(parts, axis=1), full)
    gi, gv = oracle.global_argmax(idx_max)
    assert np.array_equal(gi, np.argmax(full, axis=1))
    assert np.array_equal(gv, np.max(full, axis=1))


def test_argmax_planted_and_ties():
    V = 16032
    lg = np.zeros((6, V), dtype=np.float32)
    for row, pos in enumerate([0, 4007, 4008, 16031]):
        lg[row, pos] = 5.0
    lg[4, [100, 9000, 12000]] = 7.0       # exact tie: lowest index wins
    lg[5, :] = -1.0
    lg[5, 3] = np.nan                      # NaN never wins
    lg[5, 7] = -0.5
    idx, mx = oracle.shard_argmax(lg)
    assert list(idx) == [0, 4007, 4008, 16031, 100, 7]
    assert list(mx) == [5.0, 5.0, 5.0, 5.0, 7.0, -0.5]


def test_global_argmax_ties_to_lowest_rank():
    a = (np.array([3], dtype=np.int32), np.array([1.0], dtype=np.float32), 0)
    b = (np.array([0], dtype=np.int32), np.array([1.0], dtype=np.float32), 10)
    c = (np.array([1], dtype=np.int32), np.array([0.5], dtype=np.float32), 20)
    gi, gv = oracle.global_argmax([a, b, c])
    assert gi[0] == 3 and gv[0] == 1.0


def test_fp8_oracle_reads_the_codes_not_the_bf16_weight():
    """fp8 logits differ measurably from bf16 logits: the oracle must consume the stored bytes."""
    g = np.random.default_rng(35)
    x = synth.bf16_from_float(g.standard_normal((4, 512)))
    w = synth.bf16_normal((300, 512), 0.02, 99, 1)
    q, s = synth.quantize_e4m3_blocks(w)
    a = oracle.lm_head_logits(x, w)
    b = oracle.lm_head_logits(x, w_fp8=q, w_scale=s)
    rms = np.sqrt(np.mean(a.astype(np.float64) ** 2))
    assert np.max(np.abs(a - b)) > 0.02 * rms
    # and the dequantised weight reproduces it: dec(q) * s blockwise, then plain matmul
    deq = oracle.e4m3_to_f64(q).reshape(300, 4, 128) * s.astype(np.float64)[:, :, None]
    ref = (oracle.bf16_to_f64(x) @ deq.reshape(300, 512).T).astype(np.float32)
    assert np.max(np.abs(ref - b)) <= 1e-6 * rms


def test_lm_head_rejects_bad_chunk():
    x = np.zeros((1, 128), dtype=np.uint16)
    w = np.zeros((4, 128), dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.lm_head_logits(x, w, max_rows_per_chunk=0)
