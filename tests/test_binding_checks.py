"""The binding's tensor checks (CPU only): every bad call raises ValueError before anything is
launched. The C ABI sees only pointers and sizes, so dtype, contiguity, device and the shapes a
call implies are checked on the tensors; these tests pass host tensors, which the binding must
refuse (they are never handed to the library)."""
import os

import pytest
import torch

tt = pytest.importorskip("tensor_transformer_linear_amd")
if not os.path.exists(tt.LIB_PATH):
    pytest.skip("libtpshard.so is not built", allow_module_level=True)

bf = torch.bfloat16


def z(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


SIZES, TP, RANK = [64, 32, 32], 2, 1  # shard total 64 rows


@pytest.mark.parametrize("kw,msg", [
    (dict(x=z(16, 128), w=z(64, 120)), "w_shard has shape"),          # K differs
    (dict(x=z(16, 128), w=z(60, 128)), "w_shard has shape"),          # not the shard total
    (dict(x=z(16, 128), w=z(64, 128), b=z(63)), "bias_shard has shape"),
    (dict(x=z(16, 128, dtype=torch.float32), w=z(64, 128)), "x has dtype"),
    (dict(x=z(16, 256)[:, ::2], w=z(64, 128)), "x must be contiguous"),
    (dict(x=z(16, 128), w=z(64, 128), y=z(15, 64)), "y has shape"),    # too few rows
    (dict(x=z(16, 128), w=z(64, 128), y=z(16, 60)), "y has shape"),    # too narrow
    (dict(x=z(16, 128), w=z(64, 128), y=z(16, 64, dtype=torch.float32)), "y has dtype"),
    (dict(x=z(16, 128), w=z(64, 128), y=z(16, 64), ldy=80), "ldy"),
    (dict(x=z(16, 128), w=z(64, 128)), "must be on the GPU"),          # well formed, but host tensors
])
def test_column_linear_checks(kw, msg):
    with pytest.raises(ValueError, match=msg):
        tt.tp_column_linear(kw["x"], kw["w"], kw.get("b"), SIZES, TP, RANK, y=kw.get("y"), ldy=kw.get("ldy"))


def test_logical_output_width():
    with pytest.raises(ValueError, match="y has shape"):
        tt.tp_column_linear(z(16, 128), z(64, 128), None, SIZES, TP, RANK, y=z(16, 100),
                            layout=tt.TP_LAYOUT_LOGICAL)


@pytest.mark.parametrize("x,w,y,msg", [
    (z(16, 96), z(40, 96), None, "x_shard has shape"),     # K_logical 200, tp 2 -> K_r 100
    (z(16, 100), z(40, 96), None, "w_shard has shape"),
    (z(16, 100), z(40, 100), z(16, 40), "y_partial has dtype"),
    (z(16, 100), z(40, 100), z(16, 41, dtype=torch.float32), "y_partial has shape"),
    (z(16, 100), z(40, 100), None, "must be on the GPU"),
])
def test_row_partial_checks(x, w, y, msg):
    with pytest.raises(ValueError, match=msg):
        tt.tp_row_linear_partial(x, 200, w, None, 2, 0, y_partial=y)


@pytest.mark.parametrize("w,dt,sc,lg,msg", [
    (z(16032, 256), tt.TP_DTYPE_BF16, None, None, "w_shard has shape"),          # vocab split is 16032 rows
    (z(16000, 256), tt.TP_DTYPE_BF16, None, None, "w_shard has shape"),
    (z(16032, 256, dtype=torch.uint8), tt.TP_DTYPE_BF16, None, None, "w_shard has dtype"),
    (z(16032, 256), tt.TP_DTYPE_FP8_E4M3, None, None, "w_shard has dtype"),
    (z(16032, 256, dtype=torch.uint8), tt.TP_DTYPE_FP8_E4M3, z(16032, 3, dtype=torch.float32), None,
     "w_block_scale has shape"),
    (z(16032, 256), tt.TP_DTYPE_BF16, None, z(4, 16000, dtype=torch.float32), "logits has shape"),
])
def test_lm_head_checks(w, dt, sc, lg, msg):
    x = z(4, 256)
    if "w_shard has shape" in msg and w.shape[0] == 16032:
        x = z(4, 128)
    with pytest.raises(ValueError, match=msg):
        tt.lm_head_shard_argmax(x, 128256, 8, 0, 4008, w, dt, sc, logits=lg)


def test_lm_head_host_tensors_refused():
    with pytest.raises(ValueError, match="must be on the GPU"):
        tt.lm_head_shard_argmax(z(4, 256), 128256, 8, 0, 4008, z(16032, 256), logits=z(4, 16032, dtype=torch.float32),
                                argmax_local=z(4, dtype=torch.int32), max_logit=z(4, dtype=torch.float32),
                                workspace=z(64, dtype=torch.uint8))


def test_rmsnorm_checks():
    x, w = z(16, 128), z(64, 128)
    with pytest.raises(ValueError, match="scale has shape"):
        tt.rmsnorm_column_linear(x, z(127), 1e-6, w, None, SIZES, TP, RANK)
    with pytest.raises(ValueError, match="xnorm_out has shape"):
        tt.rmsnorm_column_linear(x, None, 1e-6, w, None, SIZES, TP, RANK, xnorm_out=z(16, 64))
    with pytest.raises(ValueError, match="workspace has dtype"):
        tt.rmsnorm_column_linear(x, None, 1e-6, w, None, SIZES, TP, RANK, workspace=z(64))
    with pytest.raises(ValueError, match="must be on the GPU"):
        tt.rmsnorm_column_linear(x, None, 1e-6, w, None, SIZES, TP, RANK, y=z(16, 64),
                                 workspace=z(1 << 16, dtype=torch.uint8))


def test_fp8_and_quantiser_checks():
    q, s = z(16, 128, dtype=torch.uint8), z(16, dtype=torch.float32)
    with pytest.raises(ValueError, match="x_scale has shape"):
        tt.tp_column_linear_fp8(q, z(15, dtype=torch.float32), z(64, 128, dtype=torch.uint8),
                                z(64, dtype=torch.float32), None, SIZES, TP, RANK)
    with pytest.raises(ValueError, match="w_scale has shape"):
        tt.tp_column_linear_fp8(q, s, z(64, 128, dtype=torch.uint8), z(32, dtype=torch.float32), None, SIZES, TP, RANK)
    with pytest.raises(ValueError, match="q has shape"):
        tt.tp_quantize_rows_e4m3(z(16, 128), q=z(16, 64, dtype=torch.uint8))
    with pytest.raises(ValueError, match="must be on the GPU"):
        tt.tp_quantize_rows_e4m3(z(16, 128), q=q, scale=s)


def test_embedding_and_fused_layer_checks():
    with pytest.raises(ValueError, match="tokens has dtype"):
        tt.tp_vocab_embedding(z(8, dtype=torch.int64), 128256, 8, 0, z(16032, 64))
    with pytest.raises(ValueError, match="table_shard has shape"):
        tt.tp_vocab_embedding(z(8, dtype=torch.int32), 128256, 8, 0, z(16000, 64))
    # heads 8, tp 2 -> 4 heads; qkv 16, ff 64 -> fph 8, qph 32, fused 24
    with pytest.raises(ValueError, match="w_qwi has shape"):
        tt.tp_qwi_swiglu(z(10, 64), 8, 0, 16, 64, 2, 0, z(120, 64), z(10, 4, 24))
    with pytest.raises(ValueError, match="y_fused has"):
        tt.tp_qwi_swiglu(z(10, 64), 8, 0, 16, 64, 2, 0, z(128, 64), z(10, 4, 20))
    with pytest.raises(ValueError, match="w_o has shape"):
        tt.tp_o_wo_partial(z(10, 96), 8, 0, 16, 64, 2, 0, z(64, 90))
    with pytest.raises(ValueError, match="partials\\[1\\] has shape"):
        tt.tp_reduce_scatter_residual([z(64, 8, dtype=torch.float32), z(60, 8, dtype=torch.float32)], 2, 32, 0,
                                      z=z(32, 8))
    with pytest.raises(ValueError, match="z has shape"):
        tt.tp_reduce_scatter_residual([z(64, 8, dtype=torch.float32)] * 2, 2, 32, 0, z=z(30, 8))
