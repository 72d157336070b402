"""Pins of the oracle's shard arithmetic (O1) and LM-head chunk rule."""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_shard_arithmetic.json")


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def test_pages_vocab_split_formula_matches_oracle():
    """Tenstorrent's padded-vocab split gives the same shard and chunks as the oracle."""
    for c in _cases():
        if "vocab" not in c:
            continue
        ndev, tile, mx = c["num_devices"], c["tile"], c["max_columns_per_device"]
        padded = math.ceil(c["vocab"] / (tile * ndev)) * tile * ndev
        size = padded // ndev
        assert padded == c["padded_vocab"] and size == c["size_per_device"]
        sizes, offs = oracle.lm_head_chunks(size, mx)
        assert sizes == c["split_sizes"]
        assert offs == [sum(sizes[:i]) for i in range(len(sizes))]
        if padded == c["vocab"]:  # no padding: the oracle's vocab shard is the page's
            for r in range(ndev):
                rows, off = oracle.vocab_shard(c["vocab"], ndev, r)
                assert rows == size and off == r * size


def test_pages_named_local_dims():
    for c in _cases():
        if "intermediate" in c:
            w, _, _, tot = oracle.shard_widths([c["intermediate"]], c["tp"], 0)
            assert w == [c["local"]] and tot == c["local"]
        if "num_heads" in c:
            head_dim = c["hidden"] // c["num_heads"]
            assert head_dim == c["head_dim"]
            w, _, _, _ = oracle.shard_widths([c["num_heads"] * head_dim], c["tp"], 0)
            assert w[0] == c["local_num_heads"] * head_dim
        if "subparam_sizes" in c:
            w, lo, lc, tot = oracle.shard_widths(c["subparam_sizes"], c["tp"], c["rank"])
            assert w == c["widths"] and tot == c["total"]


@pytest.mark.parametrize("sizes,tp", [([7], 3), ([10, 3, 3], 3), ([5, 17, 9, 4], 4), ([1], 1), ([12, 6, 6], 6),
                                      ([100, 30], 7), ([8], 8)])
def test_widths_match_array_split(sizes, tp):
    """The balanced reading equals numpy.array_split of each sub-parameter's rows."""
    pieces = [np.array_split(np.arange(sum(sizes[:i]), sum(sizes[:i + 1])), tp) for i in range(len(sizes))]
    all_rows = []
    for r in range(tp):
        w, lo, lc, tot = oracle.shard_widths(sizes, tp, r)
        want = [p[r] for p in pieces]
        assert w == [len(p) for p in want]
        assert lo == [int(p[0]) for p in want]
        assert lc == [sum(w[:i]) for i in range(len(w))]
        assert tot == sum(w)
        rows = oracle.shard_rows(sizes, tp, r)
        assert np.array_equal(rows, np.concatenate(want))
        all_rows.append(rows)
    # every logical row is owned by exactly one rank
    allr = np.sort(np.concatenate(all_rows))
    assert np.array_equal(allr, np.arange(sum(sizes)))


def test_widths_sum_to_logical_sizes_brute_force():
    for tp in range(1, 6):
        for s0 in range(tp, 14):
            for s1 in range(tp, 9):
                sizes = [s0, s1]
                tot = [0, 0]
                for r in range(tp):
                    w, _, _, _ = oracle.shard_widths(sizes, tp, r)
                    tot[0] += w[0]
                    tot[1] += w[1]
                    assert max(w[0], s0 // tp) - min(w[0], s0 // tp) <= 1
                assert tot == sizes


@pytest.mark.parametrize("sizes,tp,rank", [([3], 4, 0), ([8], 0, 0), ([8], 2, 2), ([8], 2, -1), ([], 2, 0)])
def test_widths_reject_invalid(sizes, tp, rank):
    with pytest.raises(ValueError):
        oracle.shard_widths(sizes, tp, rank)


def test_chunk_rule():
    assert oracle.lm_head_chunks(16032, 4008) == ([4008] * 4, [0, 4008, 8016, 12024])
    assert oracle.lm_head_chunks(10, 3) == ([3, 3, 3, 1], [0, 3, 6, 9])
    assert oracle.lm_head_chunks(5, 100) == ([5], [0])
    with pytest.raises(ValueError):
        oracle.lm_head_chunks(5, 0)
