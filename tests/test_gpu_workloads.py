"""The five workloads at their full sizes, through the same entry points and launch
configuration the benchmark times, checked against the oracle on sampled rows (the oracle
computes those rows one by one) and on properties that hold at any size."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tensor_transformer_linear_amd as tt
from helpers import argmax_ok, assert_close, dev_bf16, dev_f32, dev_u8, host_bits, host_f32

pytestmark = pytest.mark.gpu


def _sample_rows(M, n=48, seed=0):
    g = np.random.default_rng(seed)
    rows = set(range(0, min(8, M))) | set(range(max(0, M - 8), M)) | set(g.integers(0, M, size=n).tolist())
    return np.array(sorted(rows))


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
    sr = _sample_rows(y.shape[0], seed=2)
    ref = oracle.column_linear(inp["x"][sr], w_r, b_r, sizes, tp, rank)
    got = host_bits(y)[sr]
    assert_close(got, ref, what="local")
    assert np.array_equal(host_bits(ylog)[:, rows], host_bits(y))  # LOGICAL = LOCAL scattered, bit for bit


def test_workload3_llama8b_mlp_shard():
    c = synth.WORKLOADS[3]
    inp = synth.workload_inputs(3)
    x, wfc, wpj = inp["x"], inp["w_fc"], inp["w_proj"]
    g = tt.tp_column_linear(dev_bf16(x), dev_bf16(wfc), None, [c["inter"]], c["tp"], c["rank"], act=tt.TP_ACT_GELU_ERF)
    P = tt.tp_row_linear_partial(g, c["inter"], dev_bf16(wpj), None, c["tp"], c["rank"])
    sr = _sample_rows(x.shape[0], seed=3)
    g_ref, p_ref = oracle.mlp_rank(x[sr], wfc, wpj, rank=c["rank"])
    assert_close(host_bits(g)[sr], g_ref, what="c_fc + GELU")
    assert_close(host_f32(P)[sr], p_ref, what="c_proj partial")


def test_workload4_rmsnorm_column():
    c = synth.WORKLOADS[4]
    inp = synth.workload_inputs(4)
    x, s, w = inp["x"], inp["scale"], inp["w"]
    X, S, W = dev_bf16(x), dev_bf16(s), dev_bf16(w)
    M, K = x.shape
    y = tt.rmsnorm_column_linear(X, S, c["eps"], W, None, [c["out_logical"]], c["tp"], c["rank"])
    sr = _sample_rows(x.shape[0], n=40, seed=4)
    ref_y, ref_xn = oracle.rmsnorm_column_linear(x[sr], s, w, None, [c["out_logical"]], c["tp"], c["rank"])
    assert_close(host_bits(y)[sr], ref_y, what="materialised in the workspace")
    small = torch.empty(tt.tp_rmsnorm_workspace_min_bytes(M, K), dtype=torch.uint8, device="cuda")
    yf = tt.rmsnorm_column_linear(X, S, c["eps"], W, None, [c["out_logical"]], c["tp"], c["rank"], workspace=small)
    assert torch.equal(yf.view(torch.int16), y.view(torch.int16))
    del y, yf
    xn = torch.empty_like(X)
    y2 = tt.rmsnorm_column_linear(X, S, c["eps"], W, None, [c["out_logical"]], c["tp"], c["rank"], xnorm_out=xn)
    got_xn = host_bits(xn[torch.from_numpy(sr).cuda()])
    d = np.abs(got_xn.astype(np.int32) - ref_xn.astype(np.int32))
    assert d.max() <= 1 and np.count_nonzero(d) <= 1e-3 * d.size
    assert_close(host_bits(y2)[sr], ref_y, what="materialised")


@pytest.mark.parametrize("fp8", [False, True])
def test_workload5_lm_head(fp8):
    c = synth.WORKLOADS[5]
    inp = synth.workload_inputs(5)
    x = inp["x"]
    X = dev_bf16(x)
    if fp8:
        lg, idx, mx = tt.lm_head_shard_argmax(X, c["vocab"], c["tp"], c["rank"], c["chunk"], dev_u8(inp["w_fp8"]),
                                              tt.TP_DTYPE_FP8_E4M3, dev_f32(inp["w_scale"]))
        ref = oracle.lm_head_logits(x, w_fp8=inp["w_fp8"], w_scale=inp["w_scale"], max_rows_per_chunk=c["chunk"])
    else:
        lg, idx, mx = tt.lm_head_shard_argmax(X, c["vocab"], c["tp"], c["rank"], c["chunk"], dev_bf16(inp["w"]))
        ref = oracle.lm_head_logits(x, inp["w"], max_rows_per_chunk=c["chunk"])
    assert lg.shape == (32, 16032)
    assert_close(host_f32(lg), ref, what="logits")
    assert argmax_ok(idx.cpu().numpy(), ref) == []
