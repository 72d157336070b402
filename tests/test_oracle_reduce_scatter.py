"""Pins of the oracle's sequence-parallel reduce-scatter with residual add ([nanotron] MLP Module
c_proj output; [palm] psum_scatter and residual steps).

Pins from outside the oracle's own code: hand-listed slice rows, float32 scalar loops that add
the ranks one at a time in numpy's float32 arithmetic, torch's bf16 rounding for the residual
output, and the identity reduce-scatter = reduce, then scatter.
"""
import numpy as np
import pytest
import torch

import oracle
import synth


def _partials(tp, M, N, seed):
    return [synth.rng(70 + seed, r).standard_normal((M, N), dtype=np.float32) for r in range(tp)]


def test_slice_rows_by_hand():
    # batch 2, seq 8, tp 4: rank 1 holds positions 2, 3 of each sequence
    assert list(oracle.seq_slice_rows(2, 8, 4, 1)) == [2, 3, 10, 11]
    assert list(oracle.seq_slice_rows(1, 6, 3, 2)) == [4, 5]
    assert list(oracle.seq_slice_rows(3, 2, 1, 0)) == [0, 1, 2, 3, 4, 5]
    with pytest.raises(ValueError):
        oracle.seq_slice_rows(2, 10, 4, 0)
    with pytest.raises(ValueError):
        oracle.seq_slice_rows(2, 8, 4, 4)


def test_sum_matches_float32_scalar_loop_and_torch_rounding():
    batch, seq, tp, N = 2, 6, 3, 5
    P = _partials(tp, batch * seq, N, 1)
    res = synth.bf16_normal((batch * seq // tp, N), 1.0, 71, 9)
    for dest in range(tp):
        S, z = oracle.reduce_scatter_residual(P, batch, seq, dest, res)
        sl = seq // tp
        for b in range(batch):
            for t in range(sl):
                g, i = b * seq + dest * sl + t, b * sl + t
                for n in range(N):
                    s = np.float32(P[0][g, n])
                    for r in range(1, tp):
                        s = np.float32(s + P[r][g, n])
                    assert S[i, n] == s
                    x = torch.tensor([int(res[i, n])], dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
                    want = (torch.tensor([float(s)], dtype=torch.float32) + x.float()).to(torch.bfloat16)
                    assert int(z[i, n]) == int(want.view(torch.int16).item()) & 0xFFFF


def test_reduce_scatter_is_reduce_then_scatter():
    batch, seq, tp, N = 3, 8, 4, 7
    P = _partials(tp, batch * seq, N, 2)
    full = oracle.rank_ordered_sum(P).reshape(batch, seq, N)
    sl = seq // tp
    for dest in range(tp):
        S, z = oracle.reduce_scatter_residual(P, batch, seq, dest)
        assert z is None
        np.testing.assert_array_equal(S.reshape(batch, sl, N), full[:, dest * sl:(dest + 1) * sl])


def test_single_rank_is_the_partial_plus_residual():
    P = _partials(1, 4, 3, 3)
    res = synth.bf16_normal((4, 3), 1.0, 73, 0)
    S, z = oracle.reduce_scatter_residual(P, 2, 2, 0, res)
    np.testing.assert_array_equal(S, P[0])
    assert z.dtype == np.uint16 and z.shape == (4, 3)


def test_rank_order_is_float32_addition_order():
    # 1 + 2^-24 + 2^-24 in float32: left to right stays 1, the reverse order gives 1 + 2^-23
    big, tiny = np.float32(1.0), np.float32(2.0 ** -24)
    P = [np.full((3, 1), v, dtype=np.float32) for v in (big, tiny, tiny)]  # batch 1, seq 3, tp 3
    S, _ = oracle.reduce_scatter_residual(P, 1, 3, 0)
    assert S[0, 0] == np.float32(1.0)
    S2, _ = oracle.reduce_scatter_residual(P[::-1], 1, 3, 0)
    assert S2[0, 0] == np.float32(1.0 + 2.0 ** -23)
