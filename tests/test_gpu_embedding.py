"""Vocab-parallel embedding on the GPU against the oracle, bit for bit: small and ragged cases
with out-of-vocabulary ids, the ranks' outputs summing to the full lookup, and the prefill
size of the RMSNorm workload (32768 tokens, E 8192, vocab 128256, tp 8)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tensor_transformer_linear_amd as tt
from helpers import dev_bf16, host_bits

pytestmark = pytest.mark.gpu


def _tokens(n, vocab, seed, extra=True):
    g = np.random.default_rng(seed)
    t = g.integers(0, vocab, n).astype(np.int32)
    if extra and n >= 6:
        t[:6] = [-1, vocab, vocab + 7, 2 ** 31 - 1, -2 ** 31, 0]
    return t


@pytest.mark.parametrize("n,vocab,tp,rank,E", [(1, 50, 1, 0, 8), (333, 1003, 4, 3, 520), (64, 128256, 8, 5, 8192),
                                                (1000, 17, 3, 1, 24)])
def test_embedding_bitexact(n, vocab, tp, rank, E):
    rows, off = oracle.vocab_shard(vocab, tp, rank)
    tbl = synth.bf16_normal((rows, E), 1.0, 993, rank)
    tok = _tokens(n, vocab, n + E)
    out = tt.tp_vocab_embedding(torch.from_numpy(tok).cuda(), vocab, tp, rank, dev_bf16(tbl))
    assert np.array_equal(host_bits(out), oracle.embed_shard(tok, vocab, tp, rank, tbl))


def test_embedding_ranks_sum_to_full_lookup():
    vocab, tp, E, n = 5003, 8, 264, 2048
    full = synth.bf16_normal((vocab, E), 1.0, 994, 0)
    tok = _tokens(n, vocab, 7, extra=False)
    T = torch.from_numpy(tok).cuda()
    total = torch.zeros((n, E), dtype=torch.float32, device="cuda")
    for r in range(tp):
        rows, off = oracle.vocab_shard(vocab, tp, r)
        total += tt.tp_vocab_embedding(T, vocab, tp, r, dev_bf16(full[off:off + rows])).float()
    assert np.array_equal(total.cpu().numpy().astype(np.float64), oracle.bf16_to_f64(full[tok]))


def test_embedding_empty():
    tbl = torch.zeros((10, 8), dtype=torch.bfloat16, device="cuda")
    out = tt.tp_vocab_embedding(torch.empty(0, dtype=torch.int32, device="cuda"), 40, 4, 0, tbl)
    assert out.shape == (0, 8)


def test_embedding_prefill_size():
    vocab, tp, rank, E, n = 128256, 8, 0, 8192, 16 * 2048
    rows, off = oracle.vocab_shard(vocab, tp, rank)
    tbl = synth.bf16_normal((rows, E), 1.0, 995, 0)
    tok = _tokens(n, vocab, 8)
    out = tt.tp_vocab_embedding(torch.from_numpy(tok).cuda(), vocab, tp, rank, dev_bf16(tbl))
    assert np.array_equal(host_bits(out), oracle.embed_shard(tok, vocab, tp, rank, tbl))
