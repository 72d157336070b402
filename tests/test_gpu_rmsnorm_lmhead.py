"""GPU parity of the RMSNorm prologue and the decode LM head (through the C ABI) against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tensor_transformer_linear_amd as tt
from helpers import argmax_ok, assert_close, dev_bf16, dev_f32, dev_u8, host_bits, host_f32

pytestmark = pytest.mark.gpu


def _xnorm_agrees(got_bits, ref_bits):
    """The normalised rows equal the oracle's except where the float32 row statistic's last
    bit differs (float32 sums on the GPU, float64 in the oracle): one bf16 ulp, rarely."""
    d = np.abs(got_bits.astype(np.int32) - ref_bits.astype(np.int32))
    assert d.max() <= 1
    assert np.count_nonzero(d) <= 1e-3 * d.size


@pytest.mark.parametrize("K", [1024, 8192, 8200, 136])
@pytest.mark.parametrize("scaled", [True, False])
def test_rmsnorm_column_linear(K, scaled):
    g = np.random.default_rng(K + scaled)
    M, sizes, tp, rank = 133, [512], 4, 1
    x = synth.bf16_from_float(g.standard_normal((M, K)) * 1.3)
    s = synth.bf16_from_float(g.standard_normal(K) * 0.1) if scaled else None
    w_r = synth.bf16_from_float(g.standard_normal((128, K)) * 0.02)
    X, S, W = dev_bf16(x), (dev_bf16(s) if scaled else None), dev_bf16(w_r)
    xn = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    y_mat = tt.rmsnorm_column_linear(X, S, 1e-6, W, None, sizes, tp, rank, xnorm_out=xn)
    y_ws = tt.rmsnorm_column_linear(X, S, 1e-6, W, None, sizes, tp, rank)  # materialised in the workspace
    small = torch.empty(tt.tp_rmsnorm_workspace_min_bytes(M, K), dtype=torch.uint8, device="cuda")
    y_fused = tt.rmsnorm_column_linear(X, S, 1e-6, W, None, sizes, tp, rank, workspace=small)
    ref_y, ref_xn = oracle.rmsnorm_column_linear(x, s, w_r, None, sizes, tp, rank)
    _xnorm_agrees(host_bits(xn), ref_xn)
    # the fused A-load normalisation computes the same bf16 operand as the materialised rows
    assert torch.equal(y_mat.view(torch.int16), y_fused.view(torch.int16))
    assert torch.equal(y_mat.view(torch.int16), y_ws.view(torch.int16))
    assert_close(host_bits(y_fused), ref_y, what="rmsnorm column linear")


def test_rmsnorm_special_rows():
    K = 256
    x = np.zeros((4, K), dtype=np.uint16)
    x[1] = synth.bf16_from_float(np.where(np.arange(K) % 3 == 0, -1.0, 1.0))   # mean square 1
    x[2, 7] = synth.bf16_from_float(np.array([5.0]))[0]                          # a single non-zero
    x[3] = synth.bf16_from_float(np.full(K, 1e-3))
    zero_scale = np.zeros(K, dtype=np.uint16)
    w = synth.bf16_integers((64, K), -2, 2, 3)
    xn = torch.empty((4, K), dtype=torch.bfloat16, device="cuda")
    tt.rmsnorm_column_linear(dev_bf16(x), dev_bf16(zero_scale), 1e-6, dev_bf16(w), None, [64], 1, 0, xnorm_out=xn)
    ref, _ = oracle.rmsnorm(x, zero_scale)
    assert np.array_equal(host_bits(xn), ref)
    assert np.all(host_bits(xn)[0] == 0)


def _lm_case(B, K, vocab, tp, rank, chunk, seed, fp8):
    rows, off = oracle.vocab_shard(vocab, tp, rank)
    x = synth.bf16_normal((B, K), 1.0, 700 + seed, 0)
    w = synth.bf16_normal((rows, K), 0.02, 700 + seed, 1)
    X = dev_bf16(x)
    if fp8:
        q, s = synth.quantize_e4m3_blocks(w)
        lg, idx, mx = tt.lm_head_shard_argmax(X, vocab, tp, rank, chunk, dev_u8(q), tt.TP_DTYPE_FP8_E4M3, dev_f32(s))
        ref = oracle.lm_head_logits(x, w_fp8=q, w_scale=s, max_rows_per_chunk=chunk)
    else:
        lg, idx, mx = tt.lm_head_shard_argmax(X, vocab, tp, rank, chunk, dev_bf16(w))
        ref = oracle.lm_head_logits(x, w, max_rows_per_chunk=chunk)
    return lg, idx, mx, ref


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("B,K,vocab,tp,rank,chunk", [
    (5, 256, 1627, 8, 3, 64), (32, 384, 8 * 1000, 8, 7, 333), (1, 128, 50, 1, 0, 50), (40, 512, 3001, 2, 1, 700),
])
def test_lm_head_small(fp8, B, K, vocab, tp, rank, chunk):
    lg, idx, mx, ref = _lm_case(B, K, vocab, tp, rank, chunk, B + K, fp8)
    assert_close(host_f32(lg), ref, what="logits")
    assert argmax_ok(idx.cpu().numpy(), ref) == []
    i = idx.cpu().numpy()
    assert np.array_equal(host_f32(mx), host_f32(lg)[np.arange(B), i])


def test_lm_head_fp8_decodes_every_code_exactly():
    """One-hot x rows pick single weight columns: logits are decoded E4M3 values times
    power-of-two scales, exactly."""
    B, K, V = 32, 256, 96
    x = np.zeros((B, K), dtype=np.uint16)
    x[np.arange(B), np.arange(B) * 8] = 0x3F80
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]                     # the 254 non-NaN codes
    g = np.random.default_rng(1)
    q = g.choice(codes, size=(V, K)).astype(np.uint8)
    # the columns the one-hot rows select hold every code (V * B = 3072 slots, 254 codes)
    for v in range(V):
        q[v, np.arange(B) * 8] = codes[(v * B + np.arange(B)) % codes.size]
    s = (2.0 ** g.integers(-4, 5, size=(V, K // 128))).astype(np.float32)
    lg, idx, mx = tt.lm_head_shard_argmax(dev_bf16(x), V, 1, 0, 40, dev_u8(q), tt.TP_DTYPE_FP8_E4M3, dev_f32(s))
    ref = oracle.lm_head_logits(x, w_fp8=q, w_scale=s, max_rows_per_chunk=40)
    assert np.array_equal(host_f32(lg), ref)


def test_lm_head_planted_argmax_and_ties():
    """Maxima planted at the shard's first row, both sides of a chunk boundary and the last row;
    an exact three-way tie must resolve to the lowest index."""
    B, K, V, C = 8, 128, 16032, 4008
    ks = np.arange(B) * 16
    x = np.zeros((B, K), dtype=np.uint16)
    x[np.arange(B), ks] = 0x3F80
    w = synth.bf16_integers((V, K), -3, 3, 77)
    plant = {0: 0, 1: 4007, 2: 4008, 3: 16031, 4: 12024, 5: 8015}
    for b, pos in plant.items():
        w[pos, ks[b]] = synth.bf16_from_float(np.array([9.0]))[0]
    for pos in (100, 9000, 12000):
        w[pos, ks[6]] = synth.bf16_from_float(np.array([11.0]))[0]
    ws = tt.lm_head_workspace(B, V, 1, 0, C)
    for _ in range(3):  # the workspace is reused across calls
        lg, idx, mx = tt.lm_head_shard_argmax(dev_bf16(x), V, 1, 0, C, dev_bf16(w), workspace=ws)
        got = idx.cpu().numpy()
        for b, pos in plant.items():
            assert got[b] == pos
        assert got[6] == 100
        ref_i, ref_m = oracle.shard_argmax(oracle.lm_head_logits(x, w, max_rows_per_chunk=C))
        assert np.array_equal(got, ref_i)
        assert np.array_equal(host_f32(mx), ref_m)


def test_lm_head_chunking_does_not_change_logits():
    B, K, vocab = 16, 512, 4001
    x = synth.bf16_normal((B, K), 1.0, 801, 0)
    w = synth.bf16_normal((vocab, K), 0.02, 801, 1)
    X, W = dev_bf16(x), dev_bf16(w)
    base, bi, _ = tt.lm_head_shard_argmax(X, vocab, 1, 0, vocab, W)
    for c in (1000, 64, 63, 1):
        lg, idx, _ = tt.lm_head_shard_argmax(X, vocab, 1, 0, c, W)
        assert torch.equal(lg, base)
        assert torch.equal(idx, bi)


@pytest.mark.parametrize("shape", sorted(tt.LM_HEAD_SHAPES))
@pytest.mark.parametrize("fp8", [False, True])
def test_lm_head_every_launch_shape(shape, fp8):
    """Every launch shape of the LM head (rows per workgroup, waves, load depth) gives the
    oracle's logits and argmax; ragged chunks and a K that splits unevenly over the waves."""
    tt.set_lm_head_shape(shape)
    try:
        lg, idx, mx, ref = _lm_case(7, 640, 8 * 1000 + 13, 8, 2, 333, 50 + shape, fp8)
        assert_close(host_f32(lg), ref, what=f"shape {shape}")
        assert argmax_ok(idx.cpu().numpy(), ref) == []
    finally:
        tt.set_lm_head_shape(-1)


@pytest.mark.parametrize("shape", [8, 9])
@pytest.mark.parametrize("B,K", [(40, 256), (3, 96), (9, 200)])
def test_lm_head_lds_ring_batch_passes_and_ragged_k(shape, B, K):
    """The LDS-ring kernels over two 32-row batch passes, and with a bf16 K that their stage
    width does not divide (96 for 64-wide stages, 200 for both), where the launcher falls back
    to the register-streaming kernel."""
    tt.set_lm_head_shape(shape)
    try:
        for fp8 in ([False, True] if K % 128 == 0 else [False]):
            lg, idx, mx, ref = _lm_case(B, K, 2 * 1000 + 37, 2, 1, 500, 90 + shape, fp8)
            assert_close(host_f32(lg), ref, what=f"shape {shape} fp8 {fp8}")
            assert argmax_ok(idx.cpu().numpy(), ref) == []
    finally:
        tt.set_lm_head_shape(-1)
