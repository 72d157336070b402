"""The five workloads at their full sizes, through the same entry points and launch
configuration the benchmark times, every output compared with the oracle (which runs over the
rows in blocks) under the acceptance rules of ``helpers``: bit-equal or a checked rounding
straddle for bf16 outputs, the accumulation bound for float32 outputs, the float tolerance for
both."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tensor_transformer_linear_amd as tt
from helpers import (AbsSums, admissible_rows, argmax_ok, assert_close, check_bf16, check_f32, check_rmsnorm_rows, dev_bf16,
                     dev_f32, dev_u8, host_bits, host_f32)

pytestmark = pytest.mark.gpu

BLOCK = 1024  # oracle rows per block


def test_workload2_fused_qkv_gqa_column_shard():
    c = synth.WORKLOADS[2]
    inp = synth.workload_inputs(2)
    sizes, tp, rank = list(c["sizes"]), c["tp"], c["rank"]
    rows = oracle.shard_rows(sizes, tp, rank)
    w_r, b_r = np.ascontiguousarray(inp["w"][rows]), np.ascontiguousarray(inp["bias"][rows])
    assert w_r.shape == (768, 4096)
    X = dev_bf16(inp["x"])
    y = tt.tp_column_linear(X, dev_bf16(w_r), dev_bf16(b_r), sizes, tp, rank)
    ylog = tt.tp_column_linear(X, dev_bf16(w_r), dev_bf16(b_r), sizes, tp, rank, layout=tt.TP_LAYOUT_LOGICAL)
    yf = tt.tp_column_linear(X, dev_bf16(w_r), dev_bf16(b_r), sizes, tp, rank, y_dtype=tt.TP_DTYPE_F32)
    x = inp["x"]
    got, got32 = host_bits(y), host_f32(yf)
    sums = AbsSums.bf16(x, w_r, b_r)
    n, worst = 0, 0.0
    for r0 in range(0, x.shape[0], BLOCK):
        r1 = min(x.shape[0], r0 + BLOCK)
        v = oracle.linear_sums(x[r0:r1], w_r, b_r)
        ref = oracle.column_linear(x[r0:r1], w_r, b_r, sizes, tp, rank)
        n += check_bf16(got[r0:r1], ref, v, sums, what=f"rows {r0}:{r1}", row0=r0)
        worst = max(worst, check_f32(got32[r0:r1], v, sums.block(r0, r1), what=f"f32 rows {r0}:{r1}"))
    print(f"workload 2: {n} rounding straddles of {got.size}; largest float32 error / sum|x w| = {worst:.3g}")
    assert np.array_equal(host_bits(ylog)[:, rows], got)  # LOGICAL = LOCAL scattered, bit for bit
    assert np.array_equal(got, host_bits(yf.to(torch.bfloat16)))  # bf16 = rounding of the f32 launch


def test_workload3_llama8b_mlp_shard():
    c = synth.WORKLOADS[3]
    inp = synth.workload_inputs(3)
    x, wfc, wpj = inp["x"], inp["w_fc"], inp["w_proj"]
    g = tt.tp_column_linear(dev_bf16(x), dev_bf16(wfc), None, [c["inter"]], c["tp"], c["rank"], act=tt.TP_ACT_GELU_ERF)
    P = tt.tp_row_linear_partial(g, c["inter"], dev_bf16(wpj), None, c["tp"], c["rank"])
    g_gpu, p_gpu = host_bits(g), host_f32(P)
    sums_fc = AbsSums.bf16(x, wfc)
    wpj_abs = np.abs(oracle.bf16_to_f64(wpj))
    n = 0
    for r0 in range(0, x.shape[0], BLOCK):
        r1 = min(x.shape[0], r0 + BLOCK)
        g_ref, p_ref = oracle.mlp_rank(x[r0:r1], wfc, wpj, rank=c["rank"])
        n += check_bf16(g_gpu[r0:r1], g_ref, oracle.linear_sums(x[r0:r1], wfc), sums_fc, gelu=True,
                        what=f"c_fc + GELU rows {r0}:{r1}", row0=r0)
        # c_proj: exact sums over the oracle's GELU output; where a GELU output straddled, the
        # GPU's partial multiplied the other bf16 value, which widens that row's window
        dg = np.abs(oracle.bf16_to_f64(g_gpu[r0:r1]) - oracle.bf16_to_f64(g_ref))
        check_f32(p_gpu[r0:r1], oracle.linear_sums(g_ref, wpj), AbsSums.bf16(g_ref, wpj).block(0, r1 - r0),
                  what=f"c_proj partial rows {r0}:{r1}", ref=p_ref, extra=dg @ wpj_abs.T)
    print(f"workload 3: {n} GELU rounding straddles of {g_gpu.size}")


def test_workload4_rmsnorm_column():
    c = synth.WORKLOADS[4]
    inp = synth.workload_inputs(4)
    x, s, w = inp["x"], inp["scale"], inp["w"]
    X, S, W = dev_bf16(x), dev_bf16(s), dev_bf16(w)
    M, K = x.shape
    sub = [c["out_logical"]]
    y = tt.rmsnorm_column_linear(X, S, c["eps"], W, None, sub, c["tp"], c["rank"])  # the benchmark's path
    got = host_bits(y)
    small = torch.empty(tt.tp_rmsnorm_workspace_min_bytes(M, K), dtype=torch.uint8, device="cuda")
    yf = tt.rmsnorm_column_linear(X, S, c["eps"], W, None, sub, c["tp"], c["rank"], workspace=small)
    assert np.array_equal(host_bits(yf), got)  # fused A staging = materialised rows, bit for bit
    del yf, small
    xn = torch.empty_like(X)
    y2 = tt.rmsnorm_column_linear(X, S, c["eps"], W, None, sub, c["tp"], c["rank"], xnorm_out=xn)
    assert np.array_equal(host_bits(y2), got)
    del y2
    xn_gpu = host_bits(xn)
    del xn, X
    torch.cuda.empty_cache()
    sums_w = np.abs(oracle.bf16_to_f64(w))
    n, n_rows = 0, 0
    for r0 in range(0, M, BLOCK):
        r1 = min(M, r0 + BLOCK)
        xn_ref, other = check_rmsnorm_rows(xn_gpu[r0:r1], x[r0:r1], s, r0)
        n_rows += len(other)
        # rows whose factor took the other admissible rounding are checked against the oracle's
        # sums over the rows that rounding gives
        a = admissible_rows(xn_ref, other, x[r0:r1], s)
        v = oracle.linear_sums(a, w)
        ref = oracle.column_linear(xn_ref, w, None, sub, c["tp"], c["rank"])
        sums = AbsSums(np.abs(oracle.bf16_to_f64(a)), sums_w)
        if other:
            ref_alt = oracle.column_linear(a, w, None, sub, c["tp"], c["rank"])
            assert_close(ref_alt, ref, what="admissible factor rows")
            ref = ref_alt
        n += check_bf16(got[r0:r1], ref, v, sums, what=f"rows {r0}:{r1}")
    print(f"workload 4: {n} rounding straddles of {got.size}; {n_rows} rows took the other rounding of r")
    ref_all_tol = oracle.rmsnorm_column_linear(x[:256], s, w, None, sub, c["tp"], c["rank"])[0]
    assert_close(got[:256], ref_all_tol, what="end to end, first rows")


@pytest.mark.parametrize("fp8", [False, True])
def test_workload5_lm_head(fp8):
    c = synth.WORKLOADS[5]
    inp = synth.workload_inputs(5)
    x = inp["x"]
    X = dev_bf16(x)
    if fp8:
        lg, idx, mx = tt.lm_head_shard_argmax(X, c["vocab"], c["tp"], c["rank"], c["chunk"], dev_u8(inp["w_fp8"]),
                                              tt.TP_DTYPE_FP8_E4M3, dev_f32(inp["w_scale"]))
        v = oracle.lm_head_sums(x, w_fp8=inp["w_fp8"], w_scale=inp["w_scale"], max_rows_per_chunk=c["chunk"])
        wabs = np.abs(oracle.e4m3_to_f64(inp["w_fp8"]) * np.repeat(inp["w_scale"].astype(np.float64), 128, axis=1))
    else:
        lg, idx, mx = tt.lm_head_shard_argmax(X, c["vocab"], c["tp"], c["rank"], c["chunk"], dev_bf16(inp["w"]))
        v = oracle.lm_head_sums(x, inp["w"], max_rows_per_chunk=c["chunk"])
        wabs = np.abs(oracle.bf16_to_f64(inp["w"]))
    ref = oracle.f32(v)
    assert lg.shape == (32, 16032)
    check_f32(host_f32(lg), v, np.abs(oracle.bf16_to_f64(x)) @ wabs.T, what="logits")
    assert argmax_ok(idx.cpu().numpy(), ref) == []
    # the index and maximum are those of the logits the call wrote (numpy's argmax: lowest index)
    lgh = host_f32(lg)
    assert np.array_equal(idx.cpu().numpy(), np.argmax(lgh, axis=1))
    assert np.array_equal(mx.cpu().numpy(), lgh.max(axis=1))
