"""GPU parity of the column / row linear kernels (through the C ABI) against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tensor_transformer_linear_amd as tt
from helpers import assert_close, dev_bf16, dev_f32, host_bits, host_f32

pytestmark = pytest.mark.gpu

TILES = sorted(tt.GEMM_TILES)


PATHS = [tt.GEMM_PATH_REGISTER, tt.GEMM_PATH_DMA]


@pytest.fixture(autouse=True)
def _reset_tile():
    yield
    tt.set_gemm_tile(-1)
    tt.set_gemm_path(-1)


def _int_inputs(M, K, sizes, tp, rank, seed):
    x = synth.bf16_integers((M, K), -3, 3, seed)
    w = synth.bf16_integers((sum(sizes), K), -3, 3, seed + 1)
    b = synth.bf16_integers((sum(sizes),), -8, 8, seed + 2)
    rows = oracle.shard_rows(sizes, tp, rank)
    return x, w, b, np.ascontiguousarray(w[rows]), np.ascontiguousarray(b[rows])


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("tile", [-1] + TILES)
def test_column_linear_integer_exact_every_tile(tile, path):
    """Integer inputs make every f32 sum exact: the GPU must match the oracle bit for bit.
    Ragged M and N, a sub-parameter boundary inside tiles; K = 200 (ragged against the
    register path's 64-wide steps) or K = 224 (seven 32-wide direct-to-LDS steps)."""
    tt.set_gemm_tile(tile)
    tt.set_gemm_path(path)
    M, K, sizes, tp, rank = 301, (224 if path == tt.GEMM_PATH_DMA else 200), [300, 76, 76], 2, 1
    x, w, b, w_r, b_r = _int_inputs(M, K, sizes, tp, rank, 10 + max(tile, 0))
    X, W, B = dev_bf16(x), dev_bf16(w_r), dev_bf16(b_r)
    y = tt.tp_column_linear(X, W, B, sizes, tp, rank)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(y), oracle.column_linear(x, w_r, b_r, sizes, tp, rank))
    yf = tt.tp_column_linear(X, W, B, sizes, tp, rank, y_dtype=tt.TP_DTYPE_F32)
    assert np.array_equal(host_f32(yf), oracle.column_linear(x, w_r, b_r, sizes, tp, rank, out_dtype=oracle.OUT_F32))
    # LOGICAL layout into a wider buffer: untouched columns keep their sentinel
    ldy = sum(sizes) + 24
    ybuf = torch.full((M, ldy), -7.0, dtype=torch.bfloat16, device="cuda")
    tt.tp_column_linear(X, W, B, sizes, tp, rank, y=ybuf, layout=tt.TP_LAYOUT_LOGICAL, ldy=ldy)
    want, mask = oracle.column_linear(x, w_r, b_r, sizes, tp, rank, layout=oracle.LAYOUT_LOGICAL)
    got = host_bits(ybuf)
    assert np.array_equal(got[:, :sum(sizes)][:, mask], want[:, mask])
    sentinel = host_bits(torch.tensor([-7.0], dtype=torch.bfloat16))[0]
    assert np.all(got[:, :sum(sizes)][:, ~mask] == sentinel)
    assert np.all(got[:, sum(sizes):] == sentinel)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("tile", [-1, 0, 4, 6])
def test_column_linear_gaussian_gelu(tile, path):
    tt.set_gemm_tile(tile)
    tt.set_gemm_path(path)
    g = np.random.default_rng(5)
    M, K, sizes, tp, rank = 260, (448 if path == tt.GEMM_PATH_DMA else 456), [512, 128, 128], 8, 0
    x = synth.bf16_from_float(g.standard_normal((M, K)))
    w_r = synth.bf16_from_float(g.standard_normal((96, K)) * 0.05)
    b_r = synth.bf16_from_float(g.standard_normal(96) * 0.05)
    for act in (tt.TP_ACT_NONE, tt.TP_ACT_GELU_ERF):
        for yd in (tt.TP_DTYPE_BF16, tt.TP_DTYPE_F32):
            y = tt.tp_column_linear(dev_bf16(x), dev_bf16(w_r), dev_bf16(b_r), sizes, tp, rank, act=act, y_dtype=yd)
            got = host_bits(y) if yd == tt.TP_DTYPE_BF16 else host_f32(y)
            ref = oracle.column_linear(x, w_r, b_r, sizes, tp, rank, act=act, out_dtype=yd)
            e = assert_close(got, ref, what=f"act={act} dtype={yd}")
            # far inside the tolerance: f32 outputs differ by summation rounding only, bf16
            # outputs by at most one bf16 ulp of the largest values
            assert e < (1e-4 if yd == tt.TP_DTYPE_F32 else 1e-2)


def test_gelu_every_finite_bf16():
    """K = 8 with one unit weight: the accumulator equals the input, so the output is GELU
    of every finite bf16 value, compared with the oracle's double-precision erf."""
    allbits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    v = oracle.bf16_to_f64(allbits)
    fin = allbits[np.isfinite(v)]
    M, K = fin.size, 8
    x = np.zeros((M, K), dtype=np.uint16)
    x[:, 0] = fin
    w = np.zeros((8, K), dtype=np.uint16)
    w[:, 0] = 0x3F80  # 1.0
    y = tt.tp_column_linear(dev_bf16(x), dev_bf16(w), None, [8], 1, 0, act=tt.TP_ACT_GELU_ERF)
    got = host_bits(y)[:, 0]
    ref = oracle.column_linear(x, w, None, [8], 1, 0, act=oracle.ACT_GELU)[:, 0]
    gv, rv = oracle.bf16_to_f64(got), oracle.bf16_to_f64(ref)
    same = (got == ref) | ((gv == 0) & (rv == 0))
    # f32 erff vs double erf: at most one bf16 ulp apart, and rarely
    ulp = np.abs(got.astype(np.int32) - ref.astype(np.int32))
    assert np.all(same | (ulp <= 1)), np.nonzero(~(same | (ulp <= 1)))[0][:10]
    assert np.count_nonzero(~same) <= 0.002 * M


@pytest.mark.parametrize("path", PATHS)
def test_row_partial_integer_exact_and_rank_sum(path):
    tt.set_gemm_path(path)
    # K_r = 104: one full 64-wide step and a ragged one; K_r = 96: three 32-wide DMA steps
    M, Kl, N, tp = 130, 3 * (96 if path == tt.GEMM_PATH_DMA else 104), 200, 3
    x = synth.bf16_integers((M, Kl), -3, 3, 50)
    w = synth.bf16_integers((N, Kl), -3, 3, 51)
    b = synth.bf16_integers((N,), -8, 8, 52)
    S = torch.empty((M, N), dtype=torch.float32, device="cuda")
    parts = []
    for r in range(tp):
        cols = oracle.shard_rows([Kl], tp, r)
        xr = np.ascontiguousarray(x[:, cols])
        wr = oracle.take_row_shard(w, tp, r)
        P = tt.tp_row_linear_partial(dev_bf16(xr), Kl, dev_bf16(wr), dev_bf16(b), tp, r)
        ref = oracle.row_linear_partial(xr, wr, b, rank=r)
        assert np.array_equal(host_f32(P), ref)
        parts.append(ref)
        tt.tp_row_linear_partial(dev_bf16(xr), Kl, dev_bf16(wr), dev_bf16(b), tp, r, y_partial=S, accumulate=int(r > 0))
    assert len(parts) == tp
    full = (oracle.bf16_to_f64(x) @ oracle.bf16_to_f64(w).T + oracle.bf16_to_f64(b)).astype(np.float32)
    assert np.array_equal(host_f32(S), oracle.rank_ordered_sum(parts))
    assert np.array_equal(host_f32(S), full)


def test_mlp_gpt2_small_tp2_both_ranks():
    """GPT-2-small MLP shard, tp=2, ranks 0 and 1 emulated in turn, at full size."""
    c = synth.WORKLOADS[1]
    inp = synth.workload_inputs(1)
    x, wfc, wpj = inp["x"], inp["w_fc"], inp["w_proj"]
    X = dev_bf16(x)
    S = torch.empty((x.shape[0], c["hidden"]), dtype=torch.float32, device="cuda")
    parts = []
    for r in range(c["tp"]):
        wfc_r = oracle.take_column_shard(wfc, [c["inter"]], c["tp"], r)
        wpj_r = oracle.take_row_shard(wpj, c["tp"], r)
        g = tt.tp_column_linear(X, dev_bf16(wfc_r), None, [c["inter"]], c["tp"], r, act=tt.TP_ACT_GELU_ERF)
        P = tt.tp_row_linear_partial(g, c["inter"], dev_bf16(wpj_r), None, c["tp"], r)
        tt.tp_row_linear_partial(g, c["inter"], dev_bf16(wpj_r), None, c["tp"], r, y_partial=S, accumulate=int(r > 0))
        g_ref, p_ref = oracle.mlp_rank(x, wfc_r, wpj_r, rank=r)
        assert_close(host_bits(g), g_ref, what=f"gelu rank {r}")
        # the GPU partial is checked on its own bf16 intermediate and on the oracle's
        assert_close(host_f32(P), oracle.row_linear_partial(host_bits(g), wpj_r), what=f"partial rank {r} (gpu g)")
        assert_close(host_f32(P), p_ref, what=f"partial rank {r}")
        parts.append(p_ref)
    assert_close(host_f32(S), oracle.rank_ordered_sum(parts), what="rank sum")
    _, full = oracle.mlp_rank(x, wfc, wpj)
    assert_close(host_f32(S), full, what="rank sum vs unsharded MLP")


@pytest.mark.parametrize("path", PATHS)
def test_column_shards_assemble_bitwise_to_unsharded(path):
    """All eight ranks' LOGICAL outputs together equal the tp=1 output bit for bit (the same
    K order reaches every output element whatever the N tiling)."""
    tt.set_gemm_path(path)
    sizes, tp = [4096, 1024, 1024], 8
    M, K = 192, 4096
    g = np.random.default_rng(9)
    x = synth.bf16_from_float(g.standard_normal((M, K)))
    w = synth.bf16_normal((sum(sizes), K), 0.02, 2, 1)
    b = synth.bf16_normal((sum(sizes),), 0.02, 2, 2)
    X = dev_bf16(x)
    full = tt.tp_column_linear(X, dev_bf16(w), dev_bf16(b), [sum(sizes)], 1, 0)
    asm = torch.zeros((M, sum(sizes)), dtype=torch.bfloat16, device="cuda")
    for r in range(tp):
        rows = oracle.shard_rows(sizes, tp, r)
        tt.tp_column_linear(X, dev_bf16(w[rows]), dev_bf16(b[rows]), sizes, tp, r, y=asm,
                            layout=tt.TP_LAYOUT_LOGICAL, ldy=sum(sizes))
    assert torch.equal(asm.view(torch.int16), full.view(torch.int16))
    assert_close(host_bits(full), oracle.column_linear(x, w, b, [sum(sizes)], 1, 0), what="unsharded")


def test_empty_input():
    y = torch.full((0, 64), 1.0, dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    tt.tp_column_linear(x, w, None, [64], 1, 0, y=y)
    torch.cuda.synchronize()


def test_buffer_load_span_limit():
    """The direct-to-LDS loads of the eight-wave 256x256 tile go through buffer resources that
    reach 2^31 - 1 bytes from a tile's first row. At K = 4194272 (64-byte rows) and K = 4194240
    (the largest whole number of 64-wide pairs: 128-byte rows) a full tile's last A and B rows
    sit just inside that reach, so the forced direct-to-LDS path runs with its largest offsets;
    at K = 4194304 they do not: the forced path is refused and the automatic one falls back to
    register staging. Values in {-1, 0, 1} keep every float32 partial sum exact (|sum| < 2^24),
    so sampled outputs match the oracle bit for bit."""
    M = N = 256
    rows, cols = [0, 1, 130, 255], [0, 77, 128, 255]
    g = torch.Generator(device="cuda")
    g.manual_seed(991)
    for K, fits in ((4194272, True), (4194240, True), (4194304, False)):
        x = torch.randint(-1, 2, (M, K), generator=g, device="cuda", dtype=torch.int8).to(torch.bfloat16)
        w = torch.randint(-1, 2, (N, K), generator=g, device="cuda", dtype=torch.int8).to(torch.bfloat16)
        tt.set_gemm_tile(0)
        tt.set_gemm_path(tt.GEMM_PATH_DMA)
        if fits:
            y = tt.tp_column_linear(x, w, None, [N], 1, 0)
        else:
            with pytest.raises(RuntimeError):
                tt.tp_column_linear(x, w, None, [N], 1, 0)
            tt.set_gemm_path(tt.GEMM_PATH_AUTO)
            y = tt.tp_column_linear(x, w, None, [N], 1, 0)
        torch.cuda.synchronize()
        xs = host_bits(x[rows].contiguous())
        ws = host_bits(w[cols].contiguous())
        got = host_bits(y)[np.ix_(rows, cols)]
        assert np.array_equal(got, oracle.column_linear(xs, ws, None, [len(cols)], 1, 0)), f"K = {K}"
        del x, w, y
        torch.cuda.empty_cache()


@pytest.mark.parametrize("tile", [0, 1, 2, 3])
@pytest.mark.parametrize("K", [64, 128, 448, 1344])
def test_paired_k_rows_tile_integer_exact(tile, K):
    """The eight-wave tiles (256x256, 256x128, 128x128, 128x256) on whole 64-wide K pairs
    stage two K steps per 128-byte LDS row: one pair (the prologue's later halves reload the
    last pair), a few pairs (every issue past the end reloads it), and 21 pairs (the ring of 5
    or 10 halves wraps several times; unequal A and B halves for the non-square tiles). Ragged
    M and N, a sub-parameter boundary inside the tile, bias, GELU; bit-exact on integer
    inputs."""
    tt.set_gemm_tile(tile)
    tt.set_gemm_path(tt.GEMM_PATH_DMA)
    M, sizes, tp, rank = 301, [300, 76, 76], 2, 1
    x, w, b, w_r, b_r = _int_inputs(M, K, sizes, tp, rank, 40 + K + tile)
    y = tt.tp_column_linear(dev_bf16(x), dev_bf16(w_r), dev_bf16(b_r), sizes, tp, rank, y_dtype=tt.TP_DTYPE_F32)
    torch.cuda.synchronize()
    assert np.array_equal(host_f32(y), oracle.column_linear(x, w_r, b_r, sizes, tp, rank, out_dtype=oracle.OUT_F32))
    yg = tt.tp_column_linear(dev_bf16(x), dev_bf16(w_r), dev_bf16(b_r), sizes, tp, rank, act=tt.TP_ACT_GELU_ERF)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(yg), oracle.column_linear(x, w_r, b_r, sizes, tp, rank, act=tt.TP_ACT_GELU_ERF))
    # bf16 output without activation, with and without bias (the kernels' bf16-only output stage)
    for bias_r in (b_r, None):
        yb = tt.tp_column_linear(dev_bf16(x), dev_bf16(w_r), None if bias_r is None else dev_bf16(bias_r),
                                 sizes, tp, rank)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(yb), oracle.column_linear(x, w_r, bias_r, sizes, tp, rank))
