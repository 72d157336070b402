"""The entry points under HIP graph capture: a chain of calls captured once and replayed several times,
with eager work and synchronisations between the replays, must reproduce the eager results bit for
bit on every replay (the library records no memset, allocation or synchronisation into the graph)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tensor_transformer_linear_amd as tt
from helpers import dev_bf16

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_graph_replays_match_eager():
    dev = torch.device("cuda:0")
    M, K, inter, tp = 384, 512, 1024, 2
    x = dev_bf16(synth.bf16_normal((M, K), 1.0, 970, 0))
    wfc = [dev_bf16(synth.bf16_normal((inter // tp, K), 0.02, 970, 1 + r)) for r in range(tp)]
    wpj = [dev_bf16(synth.bf16_normal((K, inter // tp), 0.02, 970, 3 + r)) for r in range(tp)]
    # LM head (bf16), fused q_wi + SwiGLU, reduce-scatter + residual
    B, vocab, chunk = 16, 4001, 512
    xh = dev_bf16(synth.bf16_normal((B, K), 1.0, 971, 0))
    V_r, _ = oracle.vocab_shard(vocab, 2, 1)
    wh = dev_bf16(synth.bf16_normal((V_r, K), 0.02, 971, 1))
    heads, padded, qkv, ff = 4, 0, 32, 256  # fph 64, h_r 2 at tp 2
    h_r, fph, qph = oracle.qwi_dims(heads, padded, qkv, ff, tp)
    wq = dev_bf16(synth.bf16_normal((h_r * qph, K), 0.02, 972, 0))
    res = dev_bf16(synth.bf16_normal((M // tp, K), 1.0, 973, 0))
    # the eight-wave paired-row kernels: 128x128 (one ping-pong phase per K pair) and 256x256
    big = [(2048, 1024, 256), (4096, 4096, 128)]
    assert [tt.gemm_pick_tile(m, n, k) for m, n, k in big] == [2, 0]
    xb = [dev_bf16(synth.bf16_normal((m, k), 1.0, 974, i)) for i, (m, n, k) in enumerate(big)]
    wb = [dev_bf16(synth.bf16_normal((n, k), 0.02, 975, i)) for i, (m, n, k) in enumerate(big)]
    bb = [dev_bf16(synth.bf16_normal((n,), 0.1, 976, i)) for i, (m, n, k) in enumerate(big)]
    yb = [torch.empty((m, n), dtype=torch.bfloat16, device=dev) for m, n, k in big]

    g_out = [torch.empty((M, inter // tp), dtype=torch.bfloat16, device=dev) for _ in range(tp)]
    part = torch.empty((M, K), dtype=torch.float32, device=dev)
    parts = [torch.empty((M, K), dtype=torch.float32, device=dev) for _ in range(tp)]
    z = torch.empty((M // tp, K), dtype=torch.bfloat16, device=dev)
    lg = torch.empty((B, V_r), dtype=torch.float32, device=dev)
    am = torch.empty((B,), dtype=torch.int32, device=dev)
    mx = torch.empty((B,), dtype=torch.float32, device=dev)
    ws = tt.lm_head_workspace(B, vocab, 2, 1)
    yf = torch.zeros((M, h_r, qkv + fph), dtype=torch.bfloat16, device=dev)
    q = torch.empty((M, h_r, qkv), dtype=torch.bfloat16, device=dev)
    outs = g_out + [part, z, lg, am, mx, yf, q] + parts + yb

    def chain():
        for r in range(tp):
            tt.tp_column_linear(x, wfc[r], None, [inter], tp, r, act=tt.TP_ACT_GELU_ERF, y=g_out[r])
            tt.tp_row_linear_partial(g_out[r], inter, wpj[r], None, tp, r, y_partial=part, accumulate=r > 0)
            tt.tp_row_linear_partial(g_out[r], inter, wpj[r], None, tp, r, y_partial=parts[r])
        tt.tp_reduce_scatter_residual(parts, 1, M, 1, residual=res, z=z)
        tt.lm_head_shard_argmax(xh, vocab, 2, 1, chunk, wh, logits=lg, argmax_local=am, max_logit=mx, workspace=ws)
        tt.tp_qwi_swiglu(x, heads, padded, qkv, ff, tp, 0, wq, yf, q=q)
        for i, (m, n, k) in enumerate(big):
            tt.tp_column_linear(xb[i], wb[i], bb[i], [n], 1, 0, act=tt.TP_ACT_GELU_ERF if i else tt.TP_ACT_NONE, y=yb[i])

    chain()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        chain()  # warm-up on the side stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        chain()
    for rep in range(3):
        for o in outs:
            o.zero_()  # eager work between replays; every output is rewritten by the replay
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(_bits(o), _bits(e)), f"replay {rep}: output {i} differs from the eager run"
