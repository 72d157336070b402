"""Host-side tests of libtpshard: exports, shard arithmetic and argument checks (no GPU work).

Every call here either is pure host arithmetic or fails a check that the
library runs before any HIP call, so the suite runs without a GPU. Device
pointers are stand-in addresses that are never dereferenced.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle

tt = pytest.importorskip("tensor_transformer_linear_amd")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tpshard.h")

if not os.path.exists(tt.LIB_PATH):
    pytest.skip("libtpshard.so is not built", allow_module_level=True)

L = tt.lib()
A = ctypes.c_void_p(0x10000)       # 16-byte aligned stand-in device address
A2 = ctypes.c_void_p(0x20000)
A3 = ctypes.c_void_p(0x30000)
WS = ctypes.c_void_p(0x40000)      # 256-byte aligned
MIS = ctypes.c_void_p(0x10002)     # misaligned


TUNING_HEADER = os.path.join(ROOT, "tensor_transformer_linear_amd", "csrc", "tpshard_tuning.h")


def declared_functions(path=HEADER):
    text = open(path).read()
    return set(re.findall(r"^TP_API\s+[\w\s\*]+?\b(\w+)\s*\(", text, flags=re.M))


def exported_functions(path):
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True).stdout
    return {line.split()[-1] for line in out.splitlines() if " T " in line}


def test_exports_match_header():
    declared = declared_functions()
    assert {"tp_shard_widths", "tp_column_linear", "tp_row_linear_partial", "rmsnorm_column_linear",
            "lm_head_shard_argmax"} <= declared
    assert exported_functions(tt.LIB_PATH) == declared
    assert declared == set(tt.SIGNATURES)


def test_public_header_has_no_launch_switch():
    """The product ABI holds no call that selects kernels, and the library keeps no state for it:
    the launch-choice variants live in the separate tuning library only."""
    text = open(HEADER).read()
    for word in ("tp_debug", "tpt_", "set_gemm", "lm_head_shape"):
        assert word not in text, word
    src = open(os.path.join(ROOT, "tensor_transformer_linear_amd", "csrc", "tpshard_abi.hip")).read()
    assert src.count("thread_local") == 1 and "thread_local char g_err" in src


def test_tuning_library_exports():
    tuned = declared_functions(TUNING_HEADER)
    assert tuned and all(n.startswith("tpt_") for n in tuned)
    assert exported_functions(tt.TUNING_LIB_PATH) == declared_functions() | tuned
    assert tuned == {n for n in tt.TUNING_SIGNATURES if n.startswith("tpt_")}


def test_version():
    assert "gfx950" in tt.version()


@pytest.mark.parametrize("sizes,tp", [([4096, 1024, 1024], 8), ([3072], 2), ([14336], 8), ([24576], 8),
                                      ([128256], 8), ([7, 5, 5], 3), ([100, 30, 17], 7), ([9], 9), ([1], 1)])
def test_shard_widths_bit_exact_vs_oracle(sizes, tp):
    for r in range(tp):
        assert tt.tp_shard_widths(sizes, tp, r) == oracle.shard_widths(sizes, tp, r)


def test_shard_widths_configs():
    assert tt.tp_shard_widths([4096, 1024, 1024], 8, 0) == ([512, 128, 128], [0, 4096, 5120], [0, 512, 640], 768)
    assert tt.tp_shard_widths([128256], 8, 3)[1:] == ([3 * 16032], [0], 16032)


@pytest.mark.parametrize("sizes,tp,rank,status", [
    ([3], 4, 0, tt.TP_ERR_SHAPE), ([8], 0, 0, tt.TP_ERR_INVALID_ARG), ([8], 2, 2, tt.TP_ERR_INVALID_ARG),
    ([8], 2, -1, tt.TP_ERR_INVALID_ARG), ([0], 1, 0, tt.TP_ERR_INVALID_ARG), ([-4], 1, 0, tt.TP_ERR_INVALID_ARG),
    ([8] * 17, 1, 0, tt.TP_ERR_INVALID_ARG),
])
def test_shard_widths_errors(sizes, tp, rank, status):
    with pytest.raises(tt.TpError) as e:
        tt.tp_shard_widths(sizes, tp, rank)
    assert e.value.status == status and e.value.message


def _sizes(vals):
    return (ctypes.c_int64 * len(vals))(*vals)


def col(**kw):
    a = dict(x=A, M=64, K=128, w=A2, b=None, sizes=[64, 32, 32], tp=2, rank=0, act=0, y=A3, yd=0, layout=0, ldy=64)
    a.update(kw)
    s = a["sizes"]
    return L.tp_column_linear(a["x"], a["M"], a["K"], a["w"], a["b"], _sizes(s) if s is not None else None,
                              len(s) if s is not None else 1, a["tp"], a["rank"], a["act"], a["y"], a["yd"],
                              a["layout"], a["ldy"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), tt.TP_ERR_INVALID_ARG), (dict(w=None), tt.TP_ERR_INVALID_ARG), (dict(y=None), tt.TP_ERR_INVALID_ARG),
    (dict(sizes=None), tt.TP_ERR_INVALID_ARG), (dict(M=-1), tt.TP_ERR_INVALID_ARG), (dict(K=0), tt.TP_ERR_INVALID_ARG),
    (dict(K=12), tt.TP_ERR_UNSUPPORTED), (dict(tp=0), tt.TP_ERR_INVALID_ARG), (dict(rank=2), tt.TP_ERR_INVALID_ARG),
    (dict(sizes=[64, 1, 32]), tt.TP_ERR_SHAPE), (dict(act=7), tt.TP_ERR_UNSUPPORTED), (dict(yd=2), tt.TP_ERR_UNSUPPORTED),
    (dict(layout=5), tt.TP_ERR_UNSUPPORTED), (dict(ldy=56), tt.TP_ERR_SHAPE),
    (dict(layout=1, ldy=64), tt.TP_ERR_SHAPE),                 # logical width is 128
    (dict(x=MIS), tt.TP_ERR_UNSUPPORTED), (dict(y=MIS), tt.TP_ERR_UNSUPPORTED),
    (dict(b=ctypes.c_void_p(0x10001)), tt.TP_ERR_UNSUPPORTED), (dict(M=2 ** 31), tt.TP_ERR_UNSUPPORTED),
])
def test_column_linear_rejects(kw, status):
    assert col(**kw) == status
    assert L.tp_last_error().decode() != ""


def test_column_linear_empty_input_is_a_no_op():
    assert col(M=0) == tt.TP_OK
    assert L.tp_last_error().decode() == ""


def row(**kw):
    a = dict(x=A, M=16, Kl=256, N=64, w=A2, b=None, tp=2, rank=1, y=A3, acc=0)
    a.update(kw)
    return L.tp_row_linear_partial(a["x"], a["M"], a["Kl"], a["N"], a["w"], a["b"], a["tp"], a["rank"], a["y"],
                                   a["acc"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), tt.TP_ERR_INVALID_ARG), (dict(y=None), tt.TP_ERR_INVALID_ARG), (dict(N=0), tt.TP_ERR_INVALID_ARG),
    (dict(tp=0), tt.TP_ERR_INVALID_ARG), (dict(rank=5), tt.TP_ERR_INVALID_ARG), (dict(acc=2), tt.TP_ERR_INVALID_ARG),
    (dict(Kl=1), tt.TP_ERR_SHAPE), (dict(Kl=250), tt.TP_ERR_UNSUPPORTED),
    (dict(w=MIS), tt.TP_ERR_UNSUPPORTED),
])
def test_row_partial_rejects(kw, status):
    assert row(**kw) == status


def test_row_partial_empty():
    assert row(M=0) == tt.TP_OK


def rms(**kw):
    a = dict(x=A, M=8, K=128, s=None, eps=1e-6, xn=None, w=A2, sizes=[64], tp=1, rank=0, y=A3, ldy=64, ws=WS,
             wsb=1 << 20)
    a.update(kw)
    return L.rmsnorm_column_linear(a["x"], a["M"], a["K"], a["s"], a["eps"], a["xn"], a["w"], None,
                                   _sizes(a["sizes"]), len(a["sizes"]), a["tp"], a["rank"], a["y"], 0, 0, a["ldy"],
                                   a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(ws=None), tt.TP_ERR_INVALID_ARG), (dict(wsb=100), tt.TP_ERR_SHAPE), (dict(eps=-1.0), tt.TP_ERR_INVALID_ARG),
    (dict(eps=float("nan")), tt.TP_ERR_INVALID_ARG), (dict(eps=float("inf")), tt.TP_ERR_INVALID_ARG),
    (dict(ws=ctypes.c_void_p(0x40010)), tt.TP_ERR_UNSUPPORTED), (dict(s=MIS), tt.TP_ERR_UNSUPPORTED),
    (dict(xn=MIS), tt.TP_ERR_UNSUPPORTED), (dict(K=100), tt.TP_ERR_UNSUPPORTED), (dict(x=None), tt.TP_ERR_INVALID_ARG),
])
def test_rmsnorm_rejects(kw, status):
    assert rms(**kw) == status


def test_rmsnorm_workspace_size():
    assert tt.tp_rmsnorm_workspace_min_bytes(32768, 8192) == 32768 * 4 + 8192 * 2
    assert tt.tp_rmsnorm_workspace_min_bytes(3, 8) == 256 + 256
    assert tt.tp_rmsnorm_workspace_bytes(32768, 8192) == 32768 * 4 + 8192 * 2 + 32768 * 8192 * 2
    assert tt.tp_rmsnorm_workspace_bytes(3, 8) == 256 + 256 + 256


def lm(**kw):
    a = dict(x=A, B=32, K=256, vocab=1024, tp=8, rank=0, chunk=64, w=A2, wd=0, sc=None, lg=A3, am=A3, mx=None,
             ws=WS, wsb=1 << 20)
    a.update(kw)
    return L.lm_head_shard_argmax(a["x"], a["B"], a["K"], a["vocab"], a["tp"], a["rank"], a["chunk"], a["w"],
                                  a["wd"], a["sc"], a["lg"], a["am"], a["mx"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), tt.TP_ERR_INVALID_ARG), (dict(ws=None), tt.TP_ERR_INVALID_ARG), (dict(B=0), tt.TP_ERR_INVALID_ARG),
    (dict(vocab=4), tt.TP_ERR_SHAPE), (dict(chunk=0), tt.TP_ERR_SHAPE), (dict(wd=1), tt.TP_ERR_UNSUPPORTED),
    (dict(K=100), tt.TP_ERR_UNSUPPORTED), (dict(wd=2, K=192), tt.TP_ERR_UNSUPPORTED),
    (dict(wd=2, sc=None), tt.TP_ERR_INVALID_ARG), (dict(wsb=16), tt.TP_ERR_SHAPE), (dict(rank=8), tt.TP_ERR_INVALID_ARG),
    (dict(ws=ctypes.c_void_p(0x40040)), tt.TP_ERR_UNSUPPORTED), (dict(w=MIS), tt.TP_ERR_UNSUPPORTED),
])
def test_lm_head_rejects(kw, status):
    assert lm(**kw) == status


def test_lm_head_workspace_query():
    # enough for every launch shape and chunk size: 256 bytes per shard row
    assert tt.tp_lm_head_workspace_bytes(32, 128256, 8, 0) == 16032 * 256
    assert tt.tp_lm_head_workspace_bytes(100, 4001, 1, 0) == 4001 * 256
    assert tt.tp_lm_head_workspace_bytes(32, 128256, 8, 8) == 0
    assert tt.tp_lm_head_workspace_bytes(0, 128256, 8, 0) == 0


def test_tuning_choices_checked_before_anything_else():
    T = tt.tuning_lib()
    sizes = _sizes([64])
    for tile, path in ((99, -1), (-2, -1), (0, 5), (0, -2)):
        assert T.tpt_column_linear(A, 64, 128, A2, None, sizes, 1, 1, 0, 0, A3, 0, 0, 64, None, tile, path) == \
            tt.TP_ERR_INVALID_ARG
        assert b"unknown" in T.tp_last_error()
    n = T.tpt_lm_head_shape_count()
    assert n == len(tt.LM_HEAD_SHAPES)
    assert T.tpt_lm_head_shard_argmax(A, 32, 256, 4096, 8, 0, 512, A2, 0, None, A3, A, A2, WS, 1 << 20, None, n) == \
        tt.TP_ERR_INVALID_ARG
    assert tt.gemm_pick_tile(0, 1, 1) == -1
    assert tt.gemm_pick_tile(32768, 3072, 8192) in tt.GEMM_TILES


@pytest.mark.parametrize("M, N, want", [
    (32768, 3072, "256x256"), (8192, 1792, "256x256"), (8192, 4096, "256x256"),  # workload GEMMs
    (4096, 768, "128x128"), (256, 1536, "64x64"), (256, 768, "64x64"),
    (4096, 2048, "128x256"),   # 256 tiles: one full wave
    (2048, 3072, "128x256"),   # 192 tiles against 384 128x128 tiles (two waves)
    (6144, 1536, "256x256"),   # 144 tiles in one wave against 288 128x256 tiles
    (4096, 4608, "128x256"),   # 576 128x256 tiles against 1.125 waves of 256x256 tiles
    (1024, 512, "64x64"),
])
def test_gemm_tile_picker_choices(M, N, want):
    # the picker's modelled wave times (one workgroup per CU, 256 CUs, partial waves cheaper)
    bm, bn = tt.GEMM_TILES[tt.gemm_pick_tile(M, N, 4096)]
    assert f"{bm}x{bn}" == want


@pytest.mark.parametrize("M, N, want", [
    (32768, 3072, "256x256"), (4096, 4096, "256x256"), (4096, 768, "128x128"),
    (6144, 1536, "256x256"),   # 144 tiles in one wave against 576 128x128 tiles
    (2048, 3072, "128x128"),   # 384 128x128 tiles against 96 256x256 tiles
    (4096, 2048, "128x128"),
])
def test_gemm_fp8_tile_picker_choices(M, N, want):
    bm, bn = tt.GEMM_TILES[tt.gemm_fp8_pick_tile(M, N, 4096)]
    assert f"{bm}x{bn}" == want
    assert tt.gemm_fp8_pick_tile(0, 1, 1) == -1


def test_stream_probe_host_checks():
    # refused on the host before any launch (no GPU needed)
    T = tt.tuning_lib()
    assert T.tpt_stream_probe(8, 1, A, 64, A2, None) == tt.TP_ERR_SHAPE
    assert T.tpt_stream_probe(-1, 1, A, 64, A2, None) == tt.TP_ERR_SHAPE
    assert T.tpt_stream_probe(2, 1, A, 63, A2, None) == tt.TP_ERR_SHAPE
    assert T.tpt_stream_probe(2, 1, None, 64, A2, None) == tt.TP_ERR_INVALID_ARG
    assert T.tpt_stream_probe(2, 1, ctypes.c_void_p(0x40008), 64, A2, None) == tt.TP_ERR_UNSUPPORTED
    assert T.tpt_mfma_rate(0, 0, 10, A2, None) == tt.TP_ERR_SHAPE
    assert T.tpt_mfma_rate(1, 8, 0, A2, None) == tt.TP_ERR_SHAPE
    assert T.tpt_mfma_rate(0, 8, 10, None, None) == tt.TP_ERR_INVALID_ARG


def test_rmsnorm_rows_host_checks():
    # the RMSNorm-only measurement call refuses bad arguments on the host, before any launch
    T = tt.tuning_lib()
    need = tt.lib().tp_rmsnorm_workspace_min_bytes(64, 128)
    assert T.tpt_rmsnorm_rows(A, 64, 128, None, 1e-6, None, WS, need, None) == tt.TP_ERR_INVALID_ARG
    assert T.tpt_rmsnorm_rows(None, 64, 128, None, 1e-6, A2, WS, need, None) == tt.TP_ERR_INVALID_ARG
    assert T.tpt_rmsnorm_rows(A, 64, 0, None, 1e-6, A2, WS, need, None) == tt.TP_ERR_INVALID_ARG
    assert T.tpt_rmsnorm_rows(A, 64, 124, None, 1e-6, A2, WS, need, None) == tt.TP_ERR_UNSUPPORTED
    assert T.tpt_rmsnorm_rows(A, 64, 128, None, -1.0, A2, WS, need, None) == tt.TP_ERR_INVALID_ARG
    assert T.tpt_rmsnorm_rows(A, 64, 128, None, 1e-6, A2, WS, need - 1, None) == tt.TP_ERR_SHAPE
    assert b"workspace" in T.tp_last_error()
    assert T.tpt_rmsnorm_rows(A, 64, 128, None, 1e-6, ctypes.c_void_p(0x20008), WS, need, None) == \
        tt.TP_ERR_UNSUPPORTED
    assert T.tpt_rmsnorm_rows(A, 0, 128, None, 1e-6, A2, WS, need, None) == tt.TP_OK  # nothing to do


def test_tuning_routing_restores_the_product_library():
    assert getattr(tt._tls, "choices", None) is None
    with tt.tuning(tile=3):
        assert tt._tls.choices == {"tile": 3, "path": -1, "lm_shape": -1}
        with tt.tuning(lm_shape=9):
            assert tt._tls.choices["lm_shape"] == 9 and tt._tls.choices["tile"] == -1
        assert tt._tls.choices["tile"] == 3
    assert tt._tls.choices is None
    tt.set_gemm_tile(2)
    tt.set_gemm_path(1)
    tt.set_gemm_tile(-1)
    assert tt._tls.choices == {"tile": -1, "path": 1, "lm_shape": -1}
    tt.set_gemm_path(-1)
    assert tt._tls.choices is None


def test_product_path_does_not_use_the_oracle_or_generator():
    pkg_dir = os.path.dirname(tt.__file__)
    for root, _, files in os.walk(pkg_dir):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(root, f)).read()
                for word in ("import oracle", "from oracle", "import synth", "from synth", "tp_oracle"):
                    assert word not in text, (f, word)


def quant(**kw):
    a = dict(x=A, M=16, K=128, q=A2, s=A3)
    a.update(kw)
    return L.tp_quantize_rows_e4m3(a["x"], a["M"], a["K"], a["q"], a["s"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), tt.TP_ERR_INVALID_ARG), (dict(q=None), tt.TP_ERR_INVALID_ARG), (dict(s=None), tt.TP_ERR_INVALID_ARG),
    (dict(M=-1), tt.TP_ERR_INVALID_ARG), (dict(K=0), tt.TP_ERR_INVALID_ARG), (dict(K=12), tt.TP_ERR_UNSUPPORTED),
    (dict(x=MIS), tt.TP_ERR_UNSUPPORTED), (dict(q=MIS), tt.TP_ERR_UNSUPPORTED), (dict(M=2 ** 31), tt.TP_ERR_UNSUPPORTED),
])
def test_quantize_rows_rejects(kw, status):
    assert quant(**kw) == status
    assert L.tp_last_error().decode() != ""


def test_quantize_rows_empty_input_is_a_no_op():
    assert quant(M=0, x=None, q=None, s=None) == tt.TP_OK


def col8(**kw):
    a = dict(x=A, xs=A, M=64, K=128, w=A2, ws=A2, b=None, sizes=[64, 32, 32], tp=2, rank=0, act=0, y=A3, yd=0,
             layout=0, ldy=64)
    a.update(kw)
    s = a["sizes"]
    return L.tp_column_linear_fp8(a["x"], a["xs"], a["M"], a["K"], a["w"], a["ws"], a["b"], _sizes(s), len(s), a["tp"],
                                  a["rank"], a["act"], a["y"], a["yd"], a["layout"], a["ldy"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), tt.TP_ERR_INVALID_ARG), (dict(xs=None), tt.TP_ERR_INVALID_ARG), (dict(ws=None), tt.TP_ERR_INVALID_ARG),
    (dict(w=None), tt.TP_ERR_INVALID_ARG), (dict(K=96), tt.TP_ERR_UNSUPPORTED), (dict(K=12), tt.TP_ERR_UNSUPPORTED),
    (dict(sizes=[64, 1, 32]), tt.TP_ERR_SHAPE), (dict(ldy=56), tt.TP_ERR_SHAPE), (dict(rank=2), tt.TP_ERR_INVALID_ARG),
    (dict(xs=ctypes.c_void_p(0x10001)), tt.TP_ERR_UNSUPPORTED), (dict(yd=2), tt.TP_ERR_UNSUPPORTED),
])
def test_column_linear_fp8_rejects(kw, status):
    assert col8(**kw) == status
    assert L.tp_last_error().decode() != ""


def test_column_linear_fp8_empty_input_is_a_no_op():
    assert col8(M=0, x=None, xs=None, y=None) == tt.TP_OK


def emb(**kw):
    a = dict(t=A, n=64, vocab=1000, tp=4, rank=1, tbl=A2, E=128, out=A3)
    a.update(kw)
    return L.tp_vocab_embedding(a["t"], a["n"], a["vocab"], a["tp"], a["rank"], a["tbl"], a["E"], a["out"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(t=None), tt.TP_ERR_INVALID_ARG), (dict(tbl=None), tt.TP_ERR_INVALID_ARG), (dict(out=None), tt.TP_ERR_INVALID_ARG),
    (dict(n=-1), tt.TP_ERR_INVALID_ARG), (dict(tp=0), tt.TP_ERR_INVALID_ARG), (dict(rank=4), tt.TP_ERR_INVALID_ARG),
    (dict(vocab=3), tt.TP_ERR_SHAPE), (dict(E=12), tt.TP_ERR_UNSUPPORTED), (dict(out=MIS), tt.TP_ERR_UNSUPPORTED),
    (dict(E=0), tt.TP_ERR_INVALID_ARG),
])
def test_vocab_embedding_rejects(kw, status):
    assert emb(**kw) == status
    assert L.tp_last_error().decode() != ""


def test_vocab_embedding_empty_is_a_no_op():
    assert emb(n=0, t=None, out=None) == tt.TP_OK


def qwi(**kw):
    a = dict(x=A, M=64, E=256, heads=6, padded=1, qkv=32, ff=200, tp=2, rank=1, w=A2, q=A3, y=WS)
    a.update(kw)
    return L.tp_qwi_swiglu(a["x"], a["M"], a["E"], a["heads"], a["padded"], a["qkv"], a["ff"], a["tp"], a["rank"],
                           a["w"], a["q"], a["y"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), tt.TP_ERR_INVALID_ARG), (dict(w=None), tt.TP_ERR_INVALID_ARG), (dict(y=None), tt.TP_ERR_INVALID_ARG),
    (dict(tp=0), tt.TP_ERR_INVALID_ARG), (dict(rank=2), tt.TP_ERR_INVALID_ARG), (dict(heads=0), tt.TP_ERR_INVALID_ARG),
    (dict(padded=6), tt.TP_ERR_INVALID_ARG), (dict(padded=-1), tt.TP_ERR_INVALID_ARG),
    (dict(qkv=0), tt.TP_ERR_INVALID_ARG), (dict(ff=0), tt.TP_ERR_INVALID_ARG), (dict(M=-1), tt.TP_ERR_INVALID_ARG),
    (dict(E=0), tt.TP_ERR_INVALID_ARG), (dict(tp=4, rank=0), tt.TP_ERR_SHAPE), (dict(ff=4), tt.TP_ERR_SHAPE),
    (dict(E=12), tt.TP_ERR_UNSUPPORTED), (dict(q=MIS), tt.TP_ERR_UNSUPPORTED), (dict(y=MIS), tt.TP_ERR_UNSUPPORTED),
    (dict(ff=1 << 40), tt.TP_ERR_UNSUPPORTED),
])
def test_qwi_swiglu_rejects(kw, status):
    assert qwi(**kw) == status
    assert L.tp_last_error().decode() != ""


def test_qwi_swiglu_empty_is_a_no_op():
    assert qwi(M=0, x=None, y=None, q=None) == tt.TP_OK


def owo(**kw):
    # h_r = 3, fph = 40: y_fused width 3 * 72 = 216
    a = dict(y=A, M=64, heads=6, padded=1, qkv=32, ff=200, E=128, tp=2, rank=0, w=A2, out=A3, acc=0)
    a.update(kw)
    return L.tp_o_wo_partial(a["y"], a["M"], a["heads"], a["padded"], a["qkv"], a["ff"], a["E"], a["tp"], a["rank"],
                             a["w"], a["out"], a["acc"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(y=None), tt.TP_ERR_INVALID_ARG), (dict(w=None), tt.TP_ERR_INVALID_ARG), (dict(out=None), tt.TP_ERR_INVALID_ARG),
    (dict(acc=2), tt.TP_ERR_INVALID_ARG), (dict(E=0), tt.TP_ERR_INVALID_ARG), (dict(rank=-1), tt.TP_ERR_INVALID_ARG),
    (dict(heads=7), tt.TP_ERR_SHAPE), (dict(qkv=33), tt.TP_ERR_UNSUPPORTED), (dict(out=MIS), tt.TP_ERR_UNSUPPORTED),
])
def test_o_wo_partial_rejects(kw, status):
    assert owo(**kw) == status
    assert L.tp_last_error().decode() != ""


def test_o_wo_partial_empty_is_a_no_op():
    assert owo(M=0, y=None, out=None) == tt.TP_OK


def rs(**kw):
    a = dict(parts=[A, A2, A3, WS], tp=None, batch=2, seq=8, N=64, dest=1, res=A, z=A2, ys=A3)
    a.update(kw)
    parts = a["parts"]
    tp = (4 if parts is None else len(parts)) if a["tp"] is None else a["tp"]
    arr = None if parts is None else ctypes.cast((ctypes.c_void_p * max(1, len(parts)))(*parts), ctypes.c_void_p)
    return L.tp_reduce_scatter_residual(arr, tp, a["batch"], a["seq"], a["N"], a["dest"], a["res"], a["z"], a["ys"],
                                        None)


@pytest.mark.parametrize("kw,status", [
    (dict(parts=None), tt.TP_ERR_INVALID_ARG), (dict(tp=0), tt.TP_ERR_INVALID_ARG), (dict(tp=65), tt.TP_ERR_INVALID_ARG),
    (dict(dest=4), tt.TP_ERR_INVALID_ARG), (dict(dest=-1), tt.TP_ERR_INVALID_ARG), (dict(batch=-1), tt.TP_ERR_INVALID_ARG),
    (dict(seq=0), tt.TP_ERR_INVALID_ARG), (dict(N=0), tt.TP_ERR_INVALID_ARG), (dict(z=None, ys=None), tt.TP_ERR_INVALID_ARG),
    (dict(parts=[A, None, A3, WS]), tt.TP_ERR_INVALID_ARG), (dict(seq=10), tt.TP_ERR_SHAPE),
    (dict(N=66), tt.TP_ERR_UNSUPPORTED), (dict(parts=[A, MIS, A3, WS]), tt.TP_ERR_UNSUPPORTED),
    (dict(z=MIS), tt.TP_ERR_UNSUPPORTED), (dict(res=MIS), tt.TP_ERR_UNSUPPORTED),
])
def test_reduce_scatter_rejects(kw, status):
    assert rs(**kw) == status
    assert L.tp_last_error().decode() != ""


def test_reduce_scatter_rejects_oversized_grid():
    assert rs(batch=1 << 30, seq=1 << 20, N=1 << 20) == tt.TP_ERR_UNSUPPORTED


def test_reduce_scatter_empty_batch_is_a_no_op():
    assert rs(batch=0) == tt.TP_OK
    assert rs(batch=0, parts=[None, None, None, None], z=None, ys=None, res=None) == tt.TP_OK


def _llvm_tool(name):
    path = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", name)
    return path if os.path.exists(path) else None


def test_no_kernel_uses_scratch(tmp_path):
    """Every gfx950 kernel in the built library has a zero private segment. A loop-variable
    index into the kernel argument block, or a register array indexed at run time, makes the
    compiler place them in per-lane scratch memory: slower, and silent, so it is checked here
    from the code objects' own metadata."""
    objdump, readelf = _llvm_tool("llvm-objdump"), _llvm_tool("llvm-readelf")
    if objdump is None or readelf is None:
        pytest.skip("ROCm llvm tools not found")
    copy = tmp_path / "lib.so"
    copy.write_bytes(open(tt.LIB_PATH, "rb").read())
    subprocess.run([objdump, "--offloading", str(copy)], cwd=tmp_path, check=True, capture_output=True)
    sizes = {}
    for obj in sorted(tmp_path.glob("lib.so.*gfx950*")):
        notes = subprocess.run([readelf, "--notes", str(obj)], check=True, capture_output=True, text=True).stdout
        name = None
        for line in notes.splitlines():
            m = re.match(r"\s*\.name:\s+(\S+)", line)
            if m:
                name = m.group(1)
            m = re.match(r"\s*\.private_segment_fixed_size:\s+(\d+)", line)
            if m and name is not None:
                sizes[name] = int(m.group(1))
    assert len(sizes) >= 50, f"found only {len(sizes)} kernels in the code objects"
    assert {k: v for k, v in sizes.items() if v} == {}
