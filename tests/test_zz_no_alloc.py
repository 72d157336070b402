"""The allocation-free LM head (lm_head_shard_argmax_noalloc) against the entry point with a
workspace: the same logits, argmax and maxima bit for bit, on two calls in a row (the second
smaller), for bf16 and E4M3 weights; and the host-side refusal of a shard beyond its scratch."""
import numpy as np
import pytest
import torch

import synth
import tensor_transformer_linear_amd as tt
from helpers import dev_bf16, dev_f32, dev_u8

pytestmark = pytest.mark.gpu


def _inputs(B, K, vocab, tp, rank, seed):
    rows = tt.tp_shard_widths([vocab], tp, rank)[3]
    x = synth.bf16_normal((B, K), 1.0, 960 + seed, 0)
    w = synth.bf16_normal((rows, K), 0.02, 960 + seed, 1)
    q, s = synth.quantize_e4m3_blocks(w)
    return dev_bf16(x), dev_bf16(w), dev_u8(q), dev_f32(s)


@pytest.mark.parametrize("fp8", [False, True])
def test_noalloc_matches_workspace_entry_point_on_two_calls(fp8):
    # first call: the decode workload's shard shape with 48 rows (one 64-row pass); second: smaller
    for B, K, vocab, tp, rank, chunk, seed in ((48, 4096, 128256, 8, 0, 4008, 1), (5, 1024, 9001, 2, 1, 1000, 2)):
        X, W, Q, S = _inputs(B, K, vocab, tp, rank, seed)
        args = (Q, tt.TP_DTYPE_FP8_E4M3, S) if fp8 else (W, tt.TP_DTYPE_BF16, None)
        lg, idx, mx = tt.lm_head_shard_argmax(X, vocab, tp, rank, chunk, *args)
        lg2 = torch.full_like(lg, 7.0)
        idx2 = torch.full_like(idx, -1)
        mx2 = torch.full_like(mx, 7.0)
        tt.lm_head_shard_argmax_noalloc(X, vocab, tp, rank, chunk, *args, logits=lg2, argmax_local=idx2,
                                        max_logit=mx2)
        torch.cuda.synchronize()
        assert torch.equal(lg.view(torch.int32), lg2.view(torch.int32)), (B, K, vocab)
        assert torch.equal(idx, idx2) and torch.equal(mx.view(torch.int32), mx2.view(torch.int32)), (B, K, vocab)


def test_noalloc_refuses_a_shard_beyond_its_scratch():
    # 300000 rows in one shard: their candidates need more than the library's 1 MiB per GPU
    X = torch.zeros((4, 8), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((300000, 8), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(tt.TpError) as e:
        tt.lm_head_shard_argmax_noalloc(X, 300000, 1, 0, 300000, W)
    assert e.value.status == tt.TP_ERR_SHAPE and "scratch" in e.value.message
