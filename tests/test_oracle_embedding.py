"""Pins of the oracle's vocab-parallel embedding: brute force, the sum over ranks equals the
unsharded lookup, and ids outside the vocabulary give zero rows."""
import numpy as np
import pytest

import oracle
import synth


def test_embedding_brute_force():
    vocab, tp, E = 103, 4, 16
    g = np.random.default_rng(21)
    tok = g.integers(-5, vocab + 5, 200)
    for r in range(tp):
        rows, off = oracle.vocab_shard(vocab, tp, r)
        tbl = synth.bf16_normal((rows, E), 1.0, 990, r)
        out = oracle.embed_shard(tok, vocab, tp, r, tbl)
        for i, t in enumerate(tok):
            want = tbl[t - off] if (0 <= t < vocab and off <= t < off + rows) else np.zeros(E, np.uint16)
            assert np.array_equal(out[i], want)


@pytest.mark.parametrize("vocab,tp", [(128256, 8), (50257, 4), (17, 3)])
def test_embedding_ranks_sum_to_the_full_lookup(vocab, tp):
    E = 8
    full = synth.bf16_normal((vocab, E), 1.0, 991, 0)
    g = np.random.default_rng(vocab)
    tok = g.integers(0, vocab, 500)
    total = np.zeros((tok.size, E), np.float64)
    hits = np.zeros(tok.size, int)
    for r in range(tp):
        rows, off = oracle.vocab_shard(vocab, tp, r)
        out = oracle.embed_shard(tok, vocab, tp, r, full[off:off + rows])
        total += oracle.bf16_to_f64(out)
        hits += (out != 0).any(axis=1)
    assert np.array_equal(total, oracle.bf16_to_f64(full[tok]))
    assert (hits <= 1).all()  # exactly one rank holds each (non-zero) row


def test_embedding_out_of_vocab_ids_are_zero_everywhere():
    vocab, tp, E = 40, 2, 8
    tok = np.array([-1, 40, 41, 2 ** 31 - 1, -2 ** 31])
    for r in range(tp):
        rows, off = oracle.vocab_shard(vocab, tp, r)
        tbl = synth.bf16_normal((rows, E), 1.0, 992, r)
        assert not oracle.embed_shard(tok, vocab, tp, r, tbl).any()
