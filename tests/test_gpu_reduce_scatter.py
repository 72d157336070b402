"""Sequence-parallel reduce-scatter with residual add on the GPU against the oracle, bit for bit.

The kernel's arithmetic is float32 additions in rank order and one bf16 rounding, the same
operations the oracle defines, so every output must match exactly: unrolled (1, 2, 4, 8, 16)
and generic (3, 5) rank counts, every destination rank, z with and without a residual, the
float32 sum alone, a chain from the row-parallel GEMMs, and the llama-8B MLP shard's full size
(batch 8, seq 1024, hidden 4096, tp 8).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import tensor_transformer_linear_amd as tt
from helpers import dev_bf16, host_bits

pytestmark = pytest.mark.gpu


def _partials(tp, M, N, seed):
    return [synth.rng(80 + seed, r).standard_normal((M, N), dtype=np.float32) for r in range(tp)]


def _gpu(P, batch, seq, dest, res, want_z=True, want_sum=True):
    tp = len(P)
    N = P[0].shape[1]
    rows = batch * seq // tp
    parts = [torch.from_numpy(p).cuda() for p in P]
    z = torch.empty((rows, N), dtype=torch.bfloat16, device="cuda") if want_z else None
    ys = torch.empty((rows, N), dtype=torch.float32, device="cuda") if want_sum else None
    tt.tp_reduce_scatter_residual(parts, batch, seq, dest, residual=None if res is None else dev_bf16(res), z=z,
                                  y_sum=ys)
    torch.cuda.synchronize()
    return (host_bits(z) if want_z else None), (ys.cpu().numpy() if want_sum else None)


@pytest.mark.parametrize("batch,seq,tp,N", [(3, 12, 4, 20), (1, 8, 1, 64), (2, 16, 8, 136), (2, 6, 3, 8),
                                            (1, 32, 16, 32), (2, 10, 5, 12), (4, 4, 2, 4)])
def test_reduce_scatter_bitexact(batch, seq, tp, N):
    P = _partials(tp, batch * seq, N, tp * 100 + N)
    res = synth.bf16_normal((batch * seq // tp, N), 1.0, 81, tp)
    for dest in range(tp):
        S, z_ref = oracle.reduce_scatter_residual(P, batch, seq, dest, res)
        z, ys = _gpu(P, batch, seq, dest, res)
        assert np.array_equal(ys.view(np.uint32), S.view(np.uint32)), f"dest {dest}: sum differs"
        assert np.array_equal(z, z_ref), f"dest {dest}: z differs"


def test_z_without_residual_and_sum_alone():
    batch, seq, tp, N = 2, 8, 4, 48
    P = _partials(tp, batch * seq, N, 5)
    S, _ = oracle.reduce_scatter_residual(P, batch, seq, 2)
    z, _ = _gpu(P, batch, seq, 2, None, want_sum=False)
    assert np.array_equal(z, oracle.bf16_round(S))
    _, ys = _gpu(P, batch, seq, 3, None, want_z=False)
    assert np.array_equal(ys, oracle.reduce_scatter_residual(P, batch, seq, 3)[0])


def test_empty_batch():
    p = [torch.zeros((0, 8), dtype=torch.float32, device="cuda") for _ in range(2)]
    z = torch.empty((0, 8), dtype=torch.bfloat16, device="cuda")
    tt.tp_reduce_scatter_residual(p, 0, 4, 1, z=z)


def test_chain_from_row_partials():
    """c_proj row partials of every rank (GPU GEMMs) -> reduce-scatter -> residual, against the
    oracle fed with the GPU's own partials (bit-exact) and with the oracle's (tolerance)."""
    batch, seq, tp, K, N = 2, 64, 4, 512, 256
    x = synth.bf16_normal((batch * seq, K), 1.0, 82, 0)
    w = synth.bf16_normal((N, K), 0.02, 82, 1)
    res = synth.bf16_normal((batch * seq // tp, N), 1.0, 82, 2)
    parts_gpu, parts_ref = [], []
    for r in range(tp):
        xs = np.ascontiguousarray(oracle.take_row_shard(x, tp, r))
        ws = np.ascontiguousarray(oracle.take_row_shard(w, tp, r))
        parts_gpu.append(tt.tp_row_linear_partial(dev_bf16(xs), K, dev_bf16(ws), None, tp, r))
        parts_ref.append(oracle.row_linear_partial(xs, ws))
    torch.cuda.synchronize()
    own = [p.cpu().numpy() for p in parts_gpu]
    for dest in range(tp):
        z = torch.empty((batch * seq // tp, N), dtype=torch.bfloat16, device="cuda")
        tt.tp_reduce_scatter_residual(parts_gpu, batch, seq, dest, residual=dev_bf16(res), z=z)
        torch.cuda.synchronize()
        zb = host_bits(z)
        assert np.array_equal(zb, oracle.reduce_scatter_residual(own, batch, seq, dest, res)[1])
        _, z_ref = oracle.reduce_scatter_residual(parts_ref, batch, seq, dest, res)
        d = np.abs(oracle.bf16_to_f64(zb) - oracle.bf16_to_f64(z_ref))
        rf = oracle.bf16_to_f64(z_ref)
        assert d.max() <= 2e-2 * np.sqrt(np.mean(rf * rf))


def test_llama8b_mlp_full_size_every_rank():
    batch, seq, tp, N = 8, 1024, 8, 4096
    P = _partials(tp, batch * seq, N, 9)
    parts = [torch.from_numpy(p).cuda() for p in P]
    rows = batch * seq // tp
    for dest in range(tp):
        res = synth.bf16_normal((rows, N), 1.0, 83, dest)
        z = torch.empty((rows, N), dtype=torch.bfloat16, device="cuda")
        tt.tp_reduce_scatter_residual(parts, batch, seq, dest, residual=dev_bf16(res), z=z)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(z), oracle.reduce_scatter_residual(P, batch, seq, dest, res)[1]), dest
