"""GPU parity of the RMSNorm prologue and the decode LM head (through the C ABI) against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tensor_transformer_linear_amd as tt
from helpers import (AbsSums, admissible_rows, argmax_ok, assert_close, check_bf16, check_f32, check_rmsnorm_rows,
                     dev_bf16, dev_f32, dev_u8, host_bits, host_f32)

pytestmark = pytest.mark.gpu


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
    # the normalised rows: the oracle's, or rows whose factor took its other admissible rounding
    ref_xn, other = check_rmsnorm_rows(host_bits(xn), x, s)
    assert len(other) <= 2
    a = admissible_rows(ref_xn, other, x, s)
    ref_y = oracle.column_linear(a, w_r, None, sizes, tp, rank)
    check_bf16(host_bits(y_mat), ref_y, oracle.linear_sums(a, w_r), AbsSums.bf16(a, w_r), what="rmsnorm column linear")
    assert_close(host_bits(y_mat), oracle.rmsnorm_column_linear(x, s, w_r, None, sizes, tp, rank)[0], what="end to end")
    # the fused A-load normalisation computes the same bf16 operand as the materialised rows
    assert torch.equal(y_mat.view(torch.int16), y_fused.view(torch.int16))
    assert torch.equal(y_mat.view(torch.int16), y_ws.view(torch.int16))
    # the RMSNorm pass alone (the tuning library's measurement call) writes the same rows
    xn2 = torch.full((M, K), 7.0, dtype=torch.bfloat16, device="cuda")
    tt.rmsnorm_rows(X, S, 1e-6, xn2, small)
    assert torch.equal(xn.view(torch.int16), xn2.view(torch.int16))


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


@pytest.mark.parametrize("scaled", [False, True])
def test_rmsnorm_extreme_rows(scaled):
    """Rows whose squares overflow float32 (2^70, 2^100 and the largest finite bf16 next to
    ordinary values), an infinity, a NaN and a zero row: the factor r (read from the workspace)
    equals the oracle's float64 factor rounded once, bit for bit, and so do the normalised rows
    (NaN wherever the oracle has NaN: inf * 0 and NaN propagate)."""
    K = 512
    g = np.random.default_rng(9)
    x = synth.bf16_from_float(g.standard_normal((8, K)))
    x[0] = 0x6080                                        # every value 2^66: x^2 = 2^132
    x[1, 3] = 0x7180                                     # one 2^100 among N(0, 1) values
    x[2, ::2] = 0x7F7F                                   # the largest finite bf16 on every other column
    x[3, 10] = 0x7F80                                    # +inf: mean square inf, r = 0
    x[4, 20] = 0x7FC0                                    # NaN
    x[5] = 0                                             # r = f32(1 / sqrt(eps))
    x[6] = 0x0001                                        # the smallest bf16 subnormal everywhere
    s = synth.bf16_from_float(g.standard_normal(K) * 0.1) if scaled else None
    w = synth.bf16_integers((64, K), -2, 2, 4)
    M = x.shape[0]
    ws = torch.zeros(tt.tp_rmsnorm_workspace_bytes(M, K), dtype=torch.uint8, device="cuda")
    xn = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    S = dev_bf16(s) if scaled else None
    y_mat = tt.rmsnorm_column_linear(dev_bf16(x), S, 1e-6, dev_bf16(w), None, [64], 1, 0, xnorm_out=xn, workspace=ws)
    small = torch.empty(tt.tp_rmsnorm_workspace_min_bytes(M, K), dtype=torch.uint8, device="cuda")
    y_fused = tt.rmsnorm_column_linear(dev_bf16(x), S, 1e-6, dev_bf16(w), None, [64], 1, 0, workspace=small)
    torch.cuda.synchronize()
    # the fused A-load normalisation gives the materialised path's GEMM output on these rows too
    ym, yf = host_bits(y_mat), host_bits(y_fused)
    nan_m = ((ym & 0x7F80) == 0x7F80) & ((ym & 0x7F) != 0)
    nan_f = ((yf & 0x7F80) == 0x7F80) & ((yf & 0x7F) != 0)
    assert np.array_equal(nan_m, nan_f) and np.array_equal(ym[~nan_m], yf[~nan_m])
    with np.errstate(invalid="ignore", over="ignore"):
        ref, r_ref = oracle.rmsnorm(x, s)
    r_gpu = ws[:M * 4].cpu().numpy().view(np.float32)
    assert np.array_equal(r_gpu.view(np.uint32), r_ref.view(np.uint32)), (r_gpu, r_ref)
    got = host_bits(xn)
    nan_g = ((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0)
    nan_r = ((ref & 0x7F80) == 0x7F80) & ((ref & 0x7F) != 0)
    assert np.array_equal(nan_g, nan_r)
    assert np.array_equal(got[~nan_r], ref[~nan_r])


def _lm_case(B, K, vocab, tp, rank, chunk, seed, fp8):
    rows, off = oracle.vocab_shard(vocab, tp, rank)
    x = synth.bf16_normal((B, K), 1.0, 700 + seed, 0)
    w = synth.bf16_normal((rows, K), 0.02, 700 + seed, 1)
    X = dev_bf16(x)
    if fp8:
        q, s = synth.quantize_e4m3_blocks(w)
        lg, idx, mx = tt.lm_head_shard_argmax(X, vocab, tp, rank, chunk, dev_u8(q), tt.TP_DTYPE_FP8_E4M3, dev_f32(s))
        v = oracle.lm_head_sums(x, w_fp8=q, w_scale=s, max_rows_per_chunk=chunk)
        wabs = np.abs(oracle.e4m3_to_f64(q) * np.repeat(s.astype(np.float64), 128, axis=1))
    else:
        lg, idx, mx = tt.lm_head_shard_argmax(X, vocab, tp, rank, chunk, dev_bf16(w))
        v = oracle.lm_head_sums(x, w, max_rows_per_chunk=chunk)
        wabs = np.abs(oracle.bf16_to_f64(w))
    check_f32(host_f32(lg), v, np.abs(oracle.bf16_to_f64(x)) @ wabs.T, what="logits")
    return lg, idx, mx, oracle.f32(v)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("B,K,vocab,tp,rank,chunk", [
    (5, 256, 1627, 8, 3, 64), (32, 384, 8 * 1000, 8, 7, 333), (1, 128, 50, 1, 0, 50), (40, 512, 3001, 2, 1, 700),
])
def test_lm_head_small(fp8, B, K, vocab, tp, rank, chunk):
    lg, idx, mx, ref = _lm_case(B, K, vocab, tp, rank, chunk, B + K, fp8)
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
    ws = tt.lm_head_workspace(B, V, 1, 0)
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


@pytest.mark.parametrize("shape", [8, 9, 10])
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


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("B,K,vocab", [(1, 4096, 8 * 1000 + 13), (32, 1536, 2 * 700 + 1), (33, 4096, 2 * 1000 + 37),
                                       (64, 640, 8 * 333), (100, 1280, 2 * 129), (5, 128, 2 * 70)])
def test_lm_head_x_resident_slices_and_batch_passes(fp8, B, K, vocab):
    """The x-resident kernel: x slices of 1024 (32-row passes) or 512 (64-row passes) columns,
    with a ragged last slice (K = 1536, 640, 1280, 128), one 32-row pass, one 64-row pass (33 and
    64 rows), two passes (100 rows), a single row, vocab shards that end inside a 64-row tile."""
    tt.set_lm_head_shape(10)
    try:
        lg, idx, mx, ref = _lm_case(B, K, vocab, 2 if vocab % 8 else 8, 1, 500, 110 + B, fp8)
        assert argmax_ok(idx.cpu().numpy(), ref) == []
        i = idx.cpu().numpy()
        assert np.array_equal(host_f32(mx), host_f32(lg)[np.arange(B), i])
    finally:
        tt.set_lm_head_shape(-1)


@pytest.mark.parametrize("shape", [11, 12, 13, 14, 15, 16])
@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("B,K,vocab,tp", [(32, 2048, 8013, 8), (7, 4096, 201, 2), (40, 2048, 258, 2),
                                          (70, 4096, 8013, 8)])
def test_lm_head_row_quad_kernel(shape, fp8, B, K, vocab, tp):
    """The row-quad kernel at each of its slice widths, load depths and batch pass sizes (32 or
    64 rows): a full 32-row pass over a 1002-row shard (its last 64-row tile partial), a short
    batch over K 4096 (several periods of windows), 40 rows (two 32-row passes or one short
    64-row pass) over a 129-row shard (three tiles, the last holding one row), and 70 rows
    (three or two passes)."""
    tt.set_lm_head_shape(shape)
    try:
        lg, idx, mx, ref = _lm_case(B, K, vocab, tp, 1, 500, 130 + shape, fp8)
        assert argmax_ok(idx.cpu().numpy(), ref) == []
        i = idx.cpu().numpy()
        assert np.array_equal(host_f32(mx), host_f32(lg)[np.arange(B), i])
    finally:
        tt.set_lm_head_shape(-1)


@pytest.mark.parametrize("shape", [-1, 0, 9, 10, 11, 12])
@pytest.mark.parametrize("fp8", [False, True])
def test_lm_head_special_values(shape, fp8):
    """NaN and infinite inputs through every kernel family: a NaN weight row, a NaN batch row, an
    infinite x entry whose weight column holds zeros (inf * 0 = NaN), negative and positive
    values, and (bf16) infinite weights tied at two rows. The expected logits are the oracle's
    sums over the finite entries plus the non-finite products in IEEE arithmetic; the argmax
    ignores NaN, takes the lowest index among equal maxima, and gives index 0 (maximum -inf) to
    a row of NaN logits."""
    B, K, V = 4, 2048, 300
    x = synth.bf16_integers((B, K), -2, 2, 41)
    x[0, 5], x[1, 5], x[2, 5] = 0x7F80, 0, 0                 # +inf in batch row 0, column 5
    x[:3, 1] = synth.bf16_from_float(np.array([1.0, -1.0, 0.0]))
    x[3, :] = 0x7FC0                                         # a NaN batch row
    if fp8:
        g = np.random.default_rng(42)
        q = g.choice(np.array([0x30, 0x38, 0x3C, 0xB0, 0xB8, 0x00], dtype=np.uint8), size=(V, K))
        q[:, 5] = 0x38                                       # +1: row v gets +inf in batch row 0 ...
        q[:5, 5] = 0x00                                      # ... except rows 0-4 (inf * 0 = NaN)
        q[40, 5] = 0xB8                                      # -1: -inf
        q[10, 0] = 0x7F                                      # a NaN weight row
        s = (2.0 ** g.integers(-2, 3, size=(V, K // 128))).astype(np.float32)
        wd = oracle.e4m3_to_f64(q) * np.repeat(s.astype(np.float64), 128, axis=1)
        qf = q.copy()
        qf[10, 0] = 0
        finite = oracle.lm_head_sums(np.where(np.isfinite(oracle.bf16_to_f64(x)), x, 0).astype(np.uint16),
                                     w_fp8=qf, w_scale=s)
        W, dt, S = dev_u8(q), tt.TP_DTYPE_FP8_E4M3, dev_f32(s)
    else:
        w = synth.bf16_integers((V, K), -2, 2, 43)
        w[:, 5] = synth.bf16_from_float(np.ones(V))
        w[:5, 5] = 0
        w[40, 5] = synth.bf16_from_float(np.array([-1.0]))[0]
        w[10, 0] = 0x7FC0                                    # a NaN weight row
        w[[20, 250], 1] = 0x7F80                             # +inf: batch row 0 +inf (already), row 1 -inf, row 2 NaN
        w[100, 2] = 0xFF80                                   # -inf
        wd = oracle.bf16_to_f64(w)
        wf = np.where(np.isfinite(wd), w, 0).astype(np.uint16)
        finite = oracle.lm_head_sums(np.where(np.isfinite(oracle.bf16_to_f64(x)), x, 0).astype(np.uint16), wf)
        W, dt, S = dev_bf16(w), tt.TP_DTYPE_BF16, None
    xd = oracle.bf16_to_f64(x)
    ref = finite.copy()
    with np.errstate(invalid="ignore"):
        for b in range(B):
            for k in np.nonzero(~np.isfinite(xd[b]) | ~np.isfinite(wd).all(axis=0))[0]:
                special = ~np.isfinite(xd[b, k]) | ~np.isfinite(wd[:, k])
                ref[b, special] = ref[b, special] + xd[b, k] * wd[special, k]
    ref = oracle.f32(ref)
    if shape >= 0:
        tt.set_lm_head_shape(shape)
    try:
        lg, idx, mx = tt.lm_head_shard_argmax(dev_bf16(x), V, 1, 0, 128, W, dt, S)
    finally:
        tt.set_lm_head_shape(-1)
    got = host_f32(lg)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])                  # integer sums and infinities: exact
    ref_i, ref_m = oracle.shard_argmax(ref)
    assert np.array_equal(idx.cpu().numpy(), ref_i)
    assert np.array_equal(host_f32(mx), ref_m)
    assert ref_i[3] == 0 and ref_m[3] == -np.inf and ref_m[0] == np.inf


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("B,K,vocab,tp", [(1, 512, 40, 1), (3, 1024, 130, 1), (33, 2048, 1000, 2), (64, 4096, 700, 1),
                                          (65, 2048, 300, 1), (5, 1536, 300, 1)])
def test_lm_head_default_shape_edges(fp8, B, K, vocab, tp):
    """The default launch choice at its edges: one row over a shard shorter than one 64-row tile,
    33 and 64 rows (one 64-row pass), 65 rows (a second pass of one row), the smallest K the
    row-quad kernel takes (512 bf16; 1024 E4M3), and K 1536, which the E4M3 row-quad kernel does
    not take (the LDS ring runs instead)."""
    lg, idx, mx, ref = _lm_case(B, K, vocab, tp, 0, 64, 170 + B, fp8)
    assert argmax_ok(idx.cpu().numpy(), ref) == []
    i = idx.cpu().numpy()
    assert np.array_equal(host_f32(mx), host_f32(lg)[np.arange(B), i])
