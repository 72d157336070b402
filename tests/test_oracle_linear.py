"""Pins of the oracle's column / row linear, GELU and MLP against brute force and invariants."""
import json
import math
import os
import struct

import numpy as np
import pytest
import torch

import oracle
import synth


def _f32(v: float) -> float:
    """float32 rounding through the C library (struct), independent of numpy."""
    return struct.unpack("f", struct.pack("f", v))[0]


def _bf16_bits_torch(v: float) -> int:
    return int(torch.tensor([v], dtype=torch.float32).to(torch.bfloat16).view(torch.int16).item()) & 0xFFFF


def _val(bits) -> float:
    return struct.unpack("f", struct.pack("I", int(bits) << 16))[0]


def brute_column(x, w_logical, b_logical, sizes, tp, rank, gelu, out_bf16):
    """Pure-Python column linear from the unsharded weight: pick the rank's rows, loop, round."""
    # rank's rows by dealing each sub-parameter into tp contiguous pieces (larger first)
    rows = []
    base = 0
    for s in sizes:
        q, rem = divmod(s, tp)
        start = base + rank * q + min(rank, rem)
        rows += list(range(start, start + q + (1 if rank < rem else 0)))
        base += s
    M, K = x.shape
    out = []
    for m in range(M):
        line = []
        for j in rows:
            acc = 0.0
            for k in range(K):
                acc += _val(x[m, k]) * _val(w_logical[j, k])  # exact in double for these sizes
            if b_logical is not None:
                acc += _val(b_logical[j])
            a = _f32(acc)
            if gelu:
                a = _f32(0.5 * a * math.erfc(-a / math.sqrt(2.0)))
            line.append(_bf16_bits_torch(a) if out_bf16 else a)
        out.append(line)
    return np.array(out, dtype=np.uint16 if out_bf16 else np.float32), rows


@pytest.mark.parametrize("sizes,tp,rank,gelu,out_bf16,bias", [
    ([6], 1, 0, False, True, True),
    ([6, 3, 3], 3, 1, False, True, True),
    ([7, 5, 5], 2, 1, True, True, False),
    ([5, 4], 4, 3, True, False, True),
    ([9], 3, 2, False, False, False),
])
def test_column_linear_vs_brute_force(sizes, tp, rank, gelu, out_bf16, bias):
    g = np.random.default_rng(11)
    M, K = 3, 13
    x = synth.bf16_from_float(g.standard_normal((M, K)))
    w = synth.bf16_from_float(g.standard_normal((sum(sizes), K)) * 0.5)
    b = synth.bf16_from_float(g.standard_normal(sum(sizes))) if bias else None
    want, rows = brute_column(x, w, b, sizes, tp, rank, gelu, out_bf16)
    w_r = oracle.take_column_shard(w, sizes, tp, rank)
    b_r = None if b is None else b[oracle.shard_rows(sizes, tp, rank)]
    got = oracle.column_linear(x, w_r, b_r, sizes, tp, rank,
                               act=oracle.ACT_GELU if gelu else oracle.ACT_NONE,
                               out_dtype=oracle.OUT_BF16 if out_bf16 else oracle.OUT_F32)
    assert np.array_equal(got, want)
    # LOGICAL layout places each local column at its logical row index
    lg, mask = oracle.column_linear(x, w_r, b_r, sizes, tp, rank,
                                    act=oracle.ACT_GELU if gelu else oracle.ACT_NONE,
                                    out_dtype=oracle.OUT_BF16 if out_bf16 else oracle.OUT_F32,
                                    layout=oracle.LAYOUT_LOGICAL)
    assert np.array_equal(np.nonzero(mask)[0], np.array(rows))
    assert np.array_equal(lg[:, rows], want)


@pytest.mark.parametrize("sizes,tp", [([16, 8, 8], 4), ([12, 6, 6], 3), ([10], 3), ([7, 5], 2)])
def test_column_shards_concatenate_to_unsharded(sizes, tp):
    """nanotron / DeepSpeed invariant: the ranks' column shards together give the plain linear."""
    g = np.random.default_rng(2)
    M, K = 5, 24
    x = synth.bf16_from_float(g.standard_normal((M, K)))
    w = synth.bf16_from_float(g.standard_normal((sum(sizes), K)) * 0.1)
    b = synth.bf16_from_float(g.standard_normal(sum(sizes)) * 0.1)
    full = oracle.column_linear(x, w, b, [sum(sizes)], 1, 0)
    assembled = np.zeros_like(full)
    seen = np.zeros(sum(sizes), dtype=int)
    for r in range(tp):
        rows = oracle.shard_rows(sizes, tp, r)
        y, mask = oracle.column_linear(x, w[rows], b[rows], sizes, tp, r, layout=oracle.LAYOUT_LOGICAL)
        assembled[:, mask] = y[:, mask]
        seen += mask
    assert np.all(seen == 1)
    assert np.array_equal(assembled, full)
    # and the unsharded linear is the textbook x W^T + b (torch float64 matmul)
    xt = torch.from_numpy(oracle.bf16_to_f64(x))
    wt = torch.from_numpy(oracle.bf16_to_f64(w))
    bt = torch.from_numpy(oracle.bf16_to_f64(b))
    ref = (xt @ wt.T + bt).to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(full, ref)


def test_row_partials_sum_to_unsharded_exactly_on_integers():
    """Integer inputs: every partial and the rank-ordered sum are exact, so they equal x W^T bit for bit."""
    M, K, N, tp = 9, 40, 11, 4
    x = synth.bf16_integers((M, K), -3, 3, 1)
    w = synth.bf16_integers((N, K), -3, 3, 2)
    b = synth.bf16_integers((N,), -8, 8, 3)
    parts = []
    for r in range(tp):
        cols = oracle.shard_rows([K], tp, r)
        parts.append(oracle.row_linear_partial(x[:, cols], oracle.take_row_shard(w, tp, r), b, rank=r))
    s = oracle.rank_ordered_sum(parts)
    xi = oracle.bf16_to_f64(x).astype(np.int64)
    wi = oracle.bf16_to_f64(w).astype(np.int64)
    want = (xi @ wi.T + oracle.bf16_to_f64(b).astype(np.int64)[None, :]).astype(np.float32)
    assert np.array_equal(s, want)
    # only rank 0 carries the bias
    p1_nobias = oracle.row_linear_partial(x[:, oracle.shard_rows([K], tp, 1)], oracle.take_row_shard(w, tp, 1))
    assert np.array_equal(parts[1], p1_nobias)


def test_row_partial_accumulate_is_one_rounding():
    g = np.random.default_rng(4)
    x = synth.bf16_from_float(g.standard_normal((4, 32)))
    w = synth.bf16_from_float(g.standard_normal((6, 32)))
    prev = g.standard_normal((4, 6)).astype(np.float32)
    got = oracle.row_linear_partial(x, w, y_prev=prev)
    exact = oracle.bf16_to_f64(x) @ oracle.bf16_to_f64(w).T + prev.astype(np.float64)
    assert np.array_equal(got, exact.astype(np.float32))


def test_gelu_textbook_values():
    with open(os.path.join(os.path.dirname(__file__), "golden", "normal_cdf_table.json")) as f:
        t = json.load(f)
    x = np.array(t["x"], dtype=np.float32)
    got = oracle.gelu_erf(x)
    want = np.array(t["x"]) * np.array(t["phi"])
    assert np.max(np.abs(got - want)) <= t["tolerance"] * 3.0 + 1e-12
    # deep negative tail: relative accuracy (a plain 1 + erf evaluation cancels here)
    tail = t["tail"]
    xt = np.array(tail["x"], dtype=np.float32)
    want_t = np.array(tail["x"]) * np.array(tail["phi"])
    assert np.max(np.abs(oracle.gelu_erf(xt) / want_t - 1.0)) <= tail["rel_tolerance"]


def test_gelu_identities_and_libm():
    g = np.random.default_rng(5)
    a = (g.standard_normal(5000) * 4).astype(np.float32)
    ge = oracle.gelu_erf(a)
    gm = oracle.gelu_erf(-a)
    assert np.max(np.abs((ge - gm) - a.astype(np.float64))) < 1e-12
    assert oracle.gelu_erf(np.array([0.0], dtype=np.float32))[0] == 0.0
    libm = np.array([0.5 * v * math.erfc(-v / math.sqrt(2)) for v in a.astype(np.float64)])
    assert np.max(np.abs(ge - libm) / np.maximum(np.abs(libm), 1e-300)) < 1e-13
    # the tanh approximation is measurably different (guards against the wrong flavour)
    tanh = 0.5 * a * (1 + np.tanh(math.sqrt(2 / math.pi) * (a + 0.044715 * a.astype(np.float64) ** 3)))
    assert np.max(np.abs(ge - tanh)) > 1e-4


def test_gelu_is_applied_to_the_f32_accumulator_and_rounded_once():
    """A single output rounding: bf16(f32(gelu(f32(acc)))), not bf16(gelu(bf16(acc)))."""
    x = synth.bf16_from_float(np.array([[1.0, 1.0]]))
    w = synth.bf16_from_float(np.array([[0.5, 0.00390625 * 1.5]]))  # acc = 0.505859375 (9 significant bits)
    got = oracle.column_linear(x, w, None, [1], 1, 0, act=oracle.ACT_GELU)
    acc = 0.5 + 0.00390625 * 1.5
    want = _bf16_bits_torch(_f32(0.5 * acc * (1 + math.erf(acc / math.sqrt(2)))))
    assert int(got[0, 0]) == want


def test_mlp_rank_sum_equals_unsharded_mlp():
    """GELU is elementwise, so per-rank MLP partials sum to the unsharded MLP (up to f32 order)."""
    g = np.random.default_rng(6)
    M, H, F, tp = 6, 16, 24, 3
    x = synth.bf16_from_float(g.standard_normal((M, H)))
    wfc = synth.bf16_from_float(g.standard_normal((F, H)) * 0.3)
    wpj = synth.bf16_from_float(g.standard_normal((H, F)) * 0.3)
    parts = []
    for r in range(tp):
        rows = oracle.shard_rows([F], tp, r)
        _, p = oracle.mlp_rank(x, wfc[rows], oracle.take_row_shard(wpj, tp, r), rank=r)
        parts.append(p)
    s = oracle.rank_ordered_sum(parts)
    _, full = oracle.mlp_rank(x, wfc, wpj)
    assert np.max(np.abs(s - full)) <= 1e-5 * np.sqrt(np.mean(full.astype(np.float64) ** 2))
