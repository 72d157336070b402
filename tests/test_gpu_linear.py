"""GPU parity of the column / row linear kernels (through the C ABI) against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tensor_transformer_linear_amd as tt
from helpers import AbsSums, assert_close, check_bf16, check_f32, dev_bf16, dev_f32, host_bits, host_f32

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
    v = oracle.linear_sums(x, w_r, b_r)
    sums = AbsSums.bf16(x, w_r, b_r)
    for act in (tt.TP_ACT_NONE, tt.TP_ACT_GELU_ERF):
        yb = tt.tp_column_linear(dev_bf16(x), dev_bf16(w_r), dev_bf16(b_r), sizes, tp, rank, act=act)
        yf = tt.tp_column_linear(dev_bf16(x), dev_bf16(w_r), dev_bf16(b_r), sizes, tp, rank, act=act,
                                 y_dtype=tt.TP_DTYPE_F32)
        ref = oracle.column_linear(x, w_r, b_r, sizes, tp, rank, act=act)
        check_bf16(host_bits(yb), ref, v, sums, gelu=act == tt.TP_ACT_GELU_ERF, what=f"act={act} bf16")
        if act == tt.TP_ACT_NONE:
            check_f32(host_f32(yf), v, sums.block(0, M), what="f32")
        else:
            ref32 = oracle.column_linear(x, w_r, b_r, sizes, tp, rank, act=act, out_dtype=oracle.OUT_F32)
            assert assert_close(host_f32(yf), ref32, what="gelu f32") < 1e-4
        # the bf16 output is the rounding of the float32 output of the same launch settings
        assert np.array_equal(host_bits(yb), host_bits(yf.to(torch.bfloat16)))


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
    got = host_bits(y)
    ref = oracle.column_linear(x, w, None, [8], 1, 0, act=oracle.ACT_GELU)
    # the accumulator equals the input exactly: the only freedom is float32 erfc against the
    # oracle's double-precision erfc (8 float32 units), which moves a rare output by one bf16 ulp
    n = check_bf16(got, ref, oracle.linear_sums(x, w), AbsSums.bf16(x, w), gelu=True, what="every bf16 input")
    assert n <= 0.002 * got.size


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
        g_gpu = host_bits(g)
        check_bf16(g_gpu, g_ref, oracle.linear_sums(x, wfc_r), AbsSums.bf16(x, wfc_r), gelu=True,
                   what=f"gelu rank {r}")
        # the partial's exact sums are the oracle's (on its own GELU output); where a GELU output
        # straddled, the GPU's partial saw the other bf16 value: that difference widens the window
        dg = oracle.bf16_to_f64(g_gpu) - oracle.bf16_to_f64(g_ref)
        check_f32(host_f32(P), oracle.linear_sums(g_ref, wpj_r), AbsSums.bf16(g_ref, wpj_r).block(0, x.shape[0]),
                  what=f"partial rank {r}", ref=p_ref, extra=np.abs(dg) @ np.abs(oracle.bf16_to_f64(wpj_r)).T)
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
    check_bf16(host_bits(full), oracle.column_linear(x, w, b, [sum(sizes)], 1, 0), oracle.linear_sums(x, w, b),
               AbsSums.bf16(x, w, b), what="unsharded")


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
    inputs, for every output mode (bf16, bf16 + GELU, float32, float32 + GELU, float32
    accumulate)."""
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
    # float32 output with GELU: the runtime-mode output stage
    yfg = tt.tp_column_linear(dev_bf16(x), dev_bf16(w_r), dev_bf16(b_r), sizes, tp, rank, act=tt.TP_ACT_GELU_ERF,
                              y_dtype=tt.TP_DTYPE_F32)
    torch.cuda.synchronize()
    ref = oracle.column_linear(x, w_r, b_r, sizes, tp, rank, act=tt.TP_ACT_GELU_ERF, out_dtype=oracle.OUT_F32)
    assert assert_close(host_f32(yfg), ref, what="gelu f32") < 1e-4
    # bf16 output without activation, with and without bias (the kernels' bf16-only output stage)
    for bias_r in (b_r, None):
        yb = tt.tp_column_linear(dev_bf16(x), dev_bf16(w_r), None if bias_r is None else dev_bf16(bias_r),
                                 sizes, tp, rank)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(yb), oracle.column_linear(x, w_r, bias_r, sizes, tp, rank))
    # LOGICAL layout, bf16 with and without GELU: segment ends (150, 188) cut eight-column chunks, and
    # an odd row pitch leaves most rows misaligned for 16-byte stores
    ldy = sum(sizes) + 23
    for act in (tt.TP_ACT_NONE, tt.TP_ACT_GELU_ERF):
        ybuf = torch.full((M, ldy), -7.0, dtype=torch.bfloat16, device="cuda")
        tt.tp_column_linear(dev_bf16(x), dev_bf16(w_r), dev_bf16(b_r), sizes, tp, rank, act=act, y=ybuf,
                            layout=tt.TP_LAYOUT_LOGICAL, ldy=ldy)
        torch.cuda.synchronize()
        want, mask = oracle.column_linear(x, w_r, b_r, sizes, tp, rank, act=act, layout=oracle.LAYOUT_LOGICAL)
        got = host_bits(ybuf)
        sentinel = host_bits(torch.tensor([-7.0], dtype=torch.bfloat16))[0]
        assert np.array_equal(got[:, :sum(sizes)][:, mask], want[:, mask])
        assert np.all(got[:, :sum(sizes)][:, ~mask] == sentinel) and np.all(got[:, sum(sizes):] == sentinel)

    # the float32 output stage with accumulate on the same tile: a tp = 2 row-parallel pair whose
    # second rank adds onto the first's partial, bit for bit the rank-ordered sum
    N, Kl = 200, 2 * K
    xr = synth.bf16_integers((M, Kl), -3, 3, 60 + K + tile)
    wr = synth.bf16_integers((N, Kl), -3, 3, 61 + K + tile)
    br = synth.bf16_integers((N,), -8, 8, 62 + K + tile)
    S = torch.full((M, N), 5.0, dtype=torch.float32, device="cuda")
    parts = []
    for r in range(2):
        cols = oracle.shard_rows([Kl], 2, r)
        xs, ws = np.ascontiguousarray(xr[:, cols]), oracle.take_row_shard(wr, 2, r)
        tt.tp_row_linear_partial(dev_bf16(xs), Kl, dev_bf16(ws), dev_bf16(br), 2, r, y_partial=S, accumulate=r)
        parts.append(oracle.row_linear_partial(xs, ws, br, rank=r))
    torch.cuda.synchronize()
    assert np.array_equal(host_f32(S), oracle.rank_ordered_sum(parts))


@pytest.mark.parametrize("K", [512, 1024])
def test_64x64_ring_unrolled_loop_integer_exact(K):
    """The 64x64 tile's eight-stage ring runs its unrolled main loop only from 15 steps of 32 on
    (K = 512: 16 steps, one unrolled pass and a tail; K = 1024: 32 steps, three passes and a
    tail): bit-exact on integer inputs, ragged M and N, bias, both output types."""
    tt.set_gemm_tile(6)
    tt.set_gemm_path(tt.GEMM_PATH_DMA)
    M, sizes, tp, rank = 190, [300, 76, 76], 2, 1
    x, w, b, w_r, b_r = _int_inputs(M, K, sizes, tp, rank, 70 + K)
    y = tt.tp_column_linear(dev_bf16(x), dev_bf16(w_r), dev_bf16(b_r), sizes, tp, rank, y_dtype=tt.TP_DTYPE_F32)
    yb = tt.tp_column_linear(dev_bf16(x), dev_bf16(w_r), dev_bf16(b_r), sizes, tp, rank)
    torch.cuda.synchronize()
    assert np.array_equal(host_f32(y), oracle.column_linear(x, w_r, b_r, sizes, tp, rank, out_dtype=oracle.OUT_F32))
    assert np.array_equal(host_bits(yb), oracle.column_linear(x, w_r, b_r, sizes, tp, rank))


def _special_inputs(M, K, N, seed):
    """Integer-valued bf16 x and W (every finite sum exact) with IEEE special values in a few rows:
    row 0 +inf, row 1 -inf, row 2 NaN, row 3 +inf and -inf (inf - inf where both products meet),
    row 4 one product that overflows float32 (2^100 * 2^30); W's column 5 is zero for every
    third output (inf * 0 = NaN there)."""
    x = synth.bf16_integers((M, K), -3, 3, seed)
    w = synth.bf16_integers((N, K), -3, 3, seed + 1)
    w[::3, 5] = 0
    w[1::3, 5] = 0x3F80  # 1.0: nonzero where the inf lands
    w[2::3, 5] = 0xBF80  # -1.0
    w[:, 9] = 0x3F80
    w[:, 17] = 0x4E80  # 2^30
    x[0, 5] = 0x7F80      # +inf
    x[1, 5] = 0xFF80      # -inf
    x[2, 11] = 0x7FC0     # NaN
    x[3, 5], x[3, 9] = 0x7F80, 0xFF80
    x[:, 17] = 0          # the 2^30 column feeds row 4 only: every other sum stays exact in float32
    x[4, 17] = 0x7180     # 2^100
    return x, w


def _assert_special(got, want, what, finite_close=False):
    """NaN where the oracle has NaN (any NaN pattern is a correct result) and equal values
    elsewhere: infinities with their signs always, finite values bit for bit, or within the float
    tolerance with ``finite_close`` (float32 GELU: float32 erfc against the oracle's float64)."""
    if got.dtype == np.uint16:
        gnan = ((got & 0x7F80) == 0x7F80) & ((got & 0x007F) != 0)
        wnan = ((want & 0x7F80) == 0x7F80) & ((want & 0x007F) != 0)
    else:
        gnan, wnan = np.isnan(got), np.isnan(want)
    assert np.array_equal(gnan, wnan), f"{what}: NaN positions differ"
    if not finite_close:
        assert np.array_equal(got[~wnan], want[~wnan]), f"{what}: values differ"
        return
    g, w = got[~wnan], want[~wnan]
    winf = np.isinf(w)
    assert np.array_equal(g[winf], w[winf]), f"{what}: infinities differ"
    assert_close(g[~winf], w[~winf], what=what)


@pytest.mark.parametrize("tile", [-1, 0, 2, 6])
def test_column_linear_special_values(tile):
    """IEEE special values through the column GEMM and every output stage (bf16, bf16 + GELU,
    float32): infinities, NaN, inf - inf, inf * 0 and a float32 overflow, against the oracle's
    float64 arithmetic and its rounding (GELU of -inf is NaN on both sides: -inf * erfc(inf))."""
    tt.set_gemm_tile(tile)
    M, K, sizes, tp, rank = 130, 128, [300, 76, 76], 2, 1
    n_r = sum(oracle.shard_widths(sizes, tp, rank)[0])
    x, w_r = _special_inputs(M, K, n_r, 90)
    b_r = synth.bf16_integers((n_r,), -8, 8, 93)
    X, W, B = dev_bf16(x), dev_bf16(w_r), dev_bf16(b_r)
    with np.errstate(invalid="ignore", over="ignore"):
        for act in (tt.TP_ACT_NONE, tt.TP_ACT_GELU_ERF):
            y = tt.tp_column_linear(X, W, B, sizes, tp, rank, act=act)
            yf = tt.tp_column_linear(X, W, B, sizes, tp, rank, act=act, y_dtype=tt.TP_DTYPE_F32)
            torch.cuda.synchronize()
            _assert_special(host_bits(y), oracle.column_linear(x, w_r, b_r, sizes, tp, rank, act=act),
                            f"tile {tile} act {act} bf16")
            _assert_special(host_f32(yf), oracle.column_linear(x, w_r, b_r, sizes, tp, rank, act=act,
                                                               out_dtype=oracle.OUT_F32), f"tile {tile} act {act} f32",
                            finite_close=act == tt.TP_ACT_GELU_ERF)


@pytest.mark.parametrize("tile", [-1, 0, 6])
def test_row_partial_special_values_accumulate(tile):
    """The float32 partial with accumulate on special values: rank 1 adds onto rank 0's partial
    (inf + finite, inf + NaN, inf - inf across the two ranks)."""
    tt.set_gemm_tile(tile)
    M, Kl, N = 130, 256, 200
    x, w = _special_inputs(M, Kl, N, 95)
    x[5, 130], x[6, 131] = 0x7F80, 0xFF80  # rank 1's columns: +inf and -inf rows of their own
    x[0, 140] = 0xFF80                      # row 0: +inf on rank 0, -inf on rank 1
    S = torch.full((M, N), 5.0, dtype=torch.float32, device="cuda")
    parts = []
    with np.errstate(invalid="ignore", over="ignore"):
        for r in range(2):
            cols = oracle.shard_rows([Kl], 2, r)
            xs, ws = np.ascontiguousarray(x[:, cols]), oracle.take_row_shard(w, 2, r)
            tt.tp_row_linear_partial(dev_bf16(xs), Kl, dev_bf16(ws), None, 2, r, y_partial=S, accumulate=r)
            parts.append(oracle.row_linear_partial(xs, ws, None, rank=r))
        torch.cuda.synchronize()
        _assert_special(host_f32(S), oracle.rank_ordered_sum(parts), f"tile {tile} accumulate")


@pytest.mark.parametrize("M,N,want", [(2048, 3072, 3), (6144, 1536, 0), (4096, 4608, 3), (5120, 1024, 3),
                                      (1024, 9216, 0), (4096, 768, 2)])
def test_picked_tile_integer_exact(M, N, want):
    """The automatic tile on shapes where the wave-time model decides (one tile wave more or less
    than the tile-count rules would give): the launch the picker makes, bit-exact on integer
    inputs, K = 128 (two K pairs), bias and a ragged last row."""
    assert tt.gemm_pick_tile(M, N, 128) == want
    tt.set_gemm_tile(-1)
    tt.set_gemm_path(-1)
    M, K, sizes = M - 3, 128, [N]
    x, w, b, w_r, b_r = _int_inputs(M, K, sizes, 1, 0, 900 + N)
    y = tt.tp_column_linear(dev_bf16(x), dev_bf16(w_r), dev_bf16(b_r), sizes, 1, 0)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(y), oracle.column_linear(x, w_r, b_r, sizes, 1, 0))
