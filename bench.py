"""Benchmark of one tensor-parallel rank's transformer linear layers on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
  1. GPT-2-small MLP shard, tp=2: ranks 0 and 1 in turn, c_fc + GELU then the c_proj
     partial (rank 1 accumulates onto rank 0's partial: the rank-ordered sum);
  2. fused-QKV GQA column shard (sizes 4096/1024/1024, tp=8 rank 0, bias);
  3. Llama-8B MLP shard, tp=8: c_fc + GELU, c_proj float32 partial;
  4. RMSNorm (scale + 1, eps 1e-6) into a column shard [3072, 8192];
  5. vocab-sharded decode LM head (vocab 128256, tp=8 rank 0, 4 chunks of 4008 rows,
     argmax), bf16 weights and E4M3 weights with 128-wide block scales.
Every part is bracketed with HIP events on the stream its kernels run on. The headline
value is the shard-GEMM throughput: the algorithmic GEMM flops of parts 1-4 (2 M N K per
product; normalisation and activation work not counted) over those parts' time. The LM
head is reported as achieved HBM bandwidth over the bytes it must move (the weight shard
once, its scales, x and the logits). Weight copies of the LM head rotate so that every
timed call streams from HBM (the 256 MB last-level cache cannot hold the rotation).

Prints one JSON line. Inputs are seeded synthetic tensors of the workloads' shapes; they
are on the device before timing starts.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk/CU
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "shard GEMM TFLOP/s (% MFMA peak); LM-head decode GB/s (% HBM peak)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU oracle sample budget (0 = skip)")
    ap.add_argument("--parts", default="1,2,3,4,5", help="comma list of workload parts to run")
    ap.add_argument("--next", "--fp8", dest="next", type=int, default=1,
                    help="1: also time the legs beyond the five workloads: the fp8 prefill column linear, the "
                         "fused q_wi + SwiGLU and o_wo projections, the embedding and the sequence-parallel "
                         "reduce-scatter with residual (0 = skip)")
    ap.add_argument("--gemm-launches", type=int, default=0, metavar="N",
                    help="only launch each GEMM of the hot path N times in a fixed order (workloads 1-4, the fp8 "
                         "prefill GEMM, q_wi + SwiGLU and o_wo), for per-kernel profiler counters, and exit")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MB",
                    help="only run device-to-device copies of MB megabytes (the known-size kernel that "
                         "calibrates the HBM byte counters) and exit")
    ap.add_argument("--lm-shapes", default="", metavar="LIST",
                    help="only run the decode LM head (workload 5 with 32 and 64 batch rows, bf16 and E4M3 "
                         "weights) under each listed launch shape (keys of LM_HEAD_SHAPES, through the tuning "
                         "library), 25 calls each, and exit; a kernel trace of this run gives the kernel times")
    ap.add_argument("--mfma-rate", type=float, default=0.0, metavar="SECONDS",
                    help="only run the tuning library's matrix-rate probe (independent bf16 MFMAs, no memory "
                         "traffic) back to back for about SECONDS and report its TFLOP/s cold and sustained")
    ap.add_argument("--mfma-rate-workgroups", type=int, default=1024, metavar="W",
                    help="workgroups of 4 waves per --mfma-rate launch (1024: four waves per SIMD; 256: one)")
    ap.add_argument("--mfma-rate-fp8", type=int, default=0, metavar="0|1",
                    help="1: --mfma-rate runs the E4M3 instruction (v_mfma_scale_f32_32x32x64_f8f6f4)")
    ap.add_argument("--stream-probe", type=int, default=0, metavar="N",
                    help="only stream a bf16 LM-head weight shard (16032 rows x 8192 bytes, rotated copies) N "
                         "times in each fetch shape of the tuning library's probe and exit")
    return ap.parse_args()


class Workloads:
    """Device-resident inputs, weights and outputs of the five parts."""

    def __init__(self, parts, dev):
        import torch

        import synth
        import tensor_transformer_linear_amd as tt

        self.tt, self.torch, self.parts = tt, torch, parts
        W = synth.WORKLOADS

        def d16(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

        self.flops = {}
        if 1 in parts:
            c = W[1]
            inp = synth.workload_inputs(1)
            self.c1 = c
            self.x1 = d16(inp["x"])
            self.wfc1, self.wpj1 = [], []
            for r in range(c["tp"]):
                w, lo, _, tot = tt.tp_shard_widths([c["inter"]], c["tp"], r)
                self.wfc1.append(d16(inp["w_fc"][lo[0]:lo[0] + w[0]]))
                self.wpj1.append(d16(np.ascontiguousarray(inp["w_proj"][:, lo[0]:lo[0] + w[0]])))
            M = self.x1.shape[0]
            self.g1 = [torch.empty((M, self.wfc1[r].shape[0]), dtype=torch.bfloat16, device=dev) for r in range(2)]
            self.s1 = torch.empty((M, c["hidden"]), dtype=torch.float32, device=dev)
            self.flops[1] = sum(2 * M * self.wfc1[r].shape[0] * c["hidden"] * 2 for r in range(c["tp"]))
        if 2 in parts:
            c = W[2]
            inp = synth.workload_inputs(2)
            self.c2 = c
            width, lo, _, tot = tt.tp_shard_widths(list(c["sizes"]), c["tp"], c["rank"])
            rows = np.concatenate([np.arange(o, o + w) for w, o in zip(width, lo)])
            self.x2, self.w2, self.b2 = d16(inp["x"]), d16(inp["w"][rows]), d16(inp["bias"][rows])
            self.y2 = torch.empty((self.x2.shape[0], tot), dtype=torch.bfloat16, device=dev)
            self.flops[2] = 2 * self.x2.shape[0] * tot * c["hidden"]
        if 3 in parts:
            c = W[3]
            inp = synth.workload_inputs(3)
            self.c3 = c
            self.x3, self.wfc3, self.wpj3 = d16(inp["x"]), d16(inp["w_fc"]), d16(inp["w_proj"])
            M, n_r = self.x3.shape[0], self.wfc3.shape[0]
            self.g3 = torch.empty((M, n_r), dtype=torch.bfloat16, device=dev)
            self.p3 = torch.empty((M, c["hidden"]), dtype=torch.float32, device=dev)
            self.flops[3] = 2 * M * n_r * c["hidden"] * 2
        if 4 in parts:
            c = W[4]
            inp = synth.workload_inputs(4)
            self.c4 = c
            self.x4, self.s4, self.w4 = d16(inp["x"]), d16(inp["scale"]), d16(inp["w"])
            M, n_r = self.x4.shape[0], self.w4.shape[0]
            self.y4 = torch.empty((M, n_r), dtype=torch.bfloat16, device=dev)
            self.ws4 = torch.empty(tt.tp_rmsnorm_workspace_bytes(M, c["hidden"]), dtype=torch.uint8, device=dev)
            self.flops[4] = 2 * M * n_r * c["hidden"]
        if 5 in parts:
            c = W[5]
            inp = synth.workload_inputs(5)
            self.c5 = c
            self.x5 = d16(inp["x"])
            w = d16(inp["w"])
            q = torch.from_numpy(inp["w_fp8"]).to(dev)
            sc = torch.from_numpy(inp["w_scale"]).to(dev)
            # rotation: >= 512 MB of weight copies per dtype, beyond the 256 MB last-level cache
            n16 = max(2, -(-(512 << 20) // (w.numel() * 2)))
            n8 = max(2, -(-(512 << 20) // (q.numel() + sc.numel() * 4)))
            self.w5 = [w] + [w.clone() for _ in range(n16 - 1)]
            self.q5 = [(q, sc)] + [(q.clone(), sc.clone()) for _ in range(n8 - 1)]
            B, V_r = self.x5.shape[0], w.shape[0]
            self.lg5 = torch.empty((B, V_r), dtype=torch.float32, device=dev)
            self.am5 = torch.empty((B,), dtype=torch.int32, device=dev)
            self.mx5 = torch.empty((B,), dtype=torch.float32, device=dev)
            self.ws5 = tt.lm_head_workspace(B, c["vocab"], c["tp"], c["rank"], dev)
            K = c["hidden"]
            self.bytes5 = {
                "bf16": V_r * K * 2 + B * K * 2 + B * V_r * 4,
                "fp8": V_r * K + V_r * (K // 128) * 4 + B * K * 2 + B * V_r * 4,
            }
            self.rot = 0

    # --- the parts of one step -------------------------------------------------------------
    def part1(self):
        tt, c = self.tt, self.c1
        for r in range(c["tp"]):
            tt.tp_column_linear(self.x1, self.wfc1[r], None, [c["inter"]], c["tp"], r, act=tt.TP_ACT_GELU_ERF,
                                y=self.g1[r])
            tt.tp_row_linear_partial(self.g1[r], c["inter"], self.wpj1[r], None, c["tp"], r, y_partial=self.s1,
                                     accumulate=int(r > 0))

    def part2(self):
        tt, c = self.tt, self.c2
        tt.tp_column_linear(self.x2, self.w2, self.b2, list(c["sizes"]), c["tp"], c["rank"], y=self.y2)

    def part3a(self):
        tt, c = self.tt, self.c3
        tt.tp_column_linear(self.x3, self.wfc3, None, [c["inter"]], c["tp"], c["rank"], act=tt.TP_ACT_GELU_ERF,
                            y=self.g3)

    def part3b(self):
        tt, c = self.tt, self.c3
        tt.tp_row_linear_partial(self.g3, c["inter"], self.wpj3, None, c["tp"], c["rank"], y_partial=self.p3)

    def part4(self):
        tt, c = self.tt, self.c4
        tt.rmsnorm_column_linear(self.x4, self.s4, c["eps"], self.w4, None, [c["out_logical"]], c["tp"], c["rank"],
                                 y=self.y4, workspace=self.ws4)

    def part5(self, fp8):
        tt, c = self.tt, self.c5
        if fp8:
            q, sc = self.q5[self.rot % len(self.q5)]
            tt.lm_head_shard_argmax(self.x5, c["vocab"], c["tp"], c["rank"], c["chunk"], q, tt.TP_DTYPE_FP8_E4M3, sc,
                                    logits=self.lg5, argmax_local=self.am5, max_logit=self.mx5, workspace=self.ws5)
        else:
            w = self.w5[self.rot % len(self.w5)]
            tt.lm_head_shard_argmax(self.x5, c["vocab"], c["tp"], c["rank"], c["chunk"], w, logits=self.lg5,
                                    argmax_local=self.am5, max_logit=self.mx5, workspace=self.ws5)

    def segments(self):
        s = []
        if 1 in self.parts:
            s.append(("gpt2_mlp_tp2_both_ranks", self.part1))
        if 2 in self.parts:
            s.append(("qkv_gqa_column", self.part2))
        if 3 in self.parts:
            s.append(("llama8b_c_fc_gelu", self.part3a))
            s.append(("llama8b_c_proj_partial", self.part3b))
        if 4 in self.parts:
            s.append(("rmsnorm_column", self.part4))
        if 5 in self.parts:
            s.append(("lm_head_bf16", lambda: self.part5(False)))
            s.append(("lm_head_fp8", lambda: self.part5(True)))
        return s


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(budget_s: float):
    """The oracle, as it stands, on each workload of a step: workloads 1-3 and both LM heads
    in full, workload 4 on 256-row blocks of its 32768 rows (cycled) for the oracle time the
    others leave of ``budget_s`` (input generation is not timed). Returns the headline (the
    GEMM TFLOP/s of workloads 1-4, workload 4 scaled from its sample) with one entry per
    workload."""
    import oracle
    import synth

    try:
        from threadpoolctl import threadpool_info

        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    W = synth.WORKLOADS
    per = []
    t_all = time.perf_counter()

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    # workload 1: both ranks of the GPT-2 MLP shard and their rank-ordered sum
    c = W[1]
    inp = synth.workload_inputs(1)
    shards = [(oracle.take_column_shard(inp["w_fc"], [c["inter"]], c["tp"], r),
               oracle.take_row_shard(inp["w_proj"], c["tp"], r)) for r in range(c["tp"])]

    def wl1():
        parts = [oracle.mlp_rank(inp["x"], a, b, rank=r)[1] for r, (a, b) in enumerate(shards)]
        oracle.rank_ordered_sum(parts)
    m = inp["x"].shape[0]
    per.append((1, 2.0 * m * c["inter"] // c["tp"] * c["hidden"] * 2 * c["tp"], timed(wl1), "both ranks, full"))
    # workload 2: the fused-QKV column shard with bias
    c = W[2]
    inp = synth.workload_inputs(2)
    rows = oracle.shard_rows(list(c["sizes"]), c["tp"], c["rank"])
    w2, b2 = np.ascontiguousarray(inp["w"][rows]), np.ascontiguousarray(inp["bias"][rows])
    per.append((2, 2.0 * inp["x"].shape[0] * len(rows) * c["hidden"],
                timed(lambda: oracle.column_linear(inp["x"], w2, b2, list(c["sizes"]), c["tp"], c["rank"])), "full"))
    # workload 3: the Llama-8B MLP shard
    c = W[3]
    inp = synth.workload_inputs(3)
    per.append((3, 2.0 * inp["x"].shape[0] * inp["w_fc"].shape[0] * c["hidden"] * 2,
                timed(lambda: oracle.mlp_rank(inp["x"], inp["w_fc"], inp["w_proj"], rank=c["rank"])), "full"))
    # workload 5: the LM head, bf16 and E4M3 weights (GB/s over the bytes the method moves)
    c = W[5]
    inp = synth.workload_inputs(5)
    B, K = inp["x"].shape
    V = inp["w"].shape[0]
    lm = []
    for dt, nbytes, fn in (
            ("bf16", V * K * 2 + B * K * 2 + B * V * 4,
             lambda: oracle.shard_argmax(oracle.lm_head_logits(inp["x"], inp["w"], max_rows_per_chunk=c["chunk"]))),
            ("fp8", V * K + V * (K // 128) * 4 + B * K * 2 + B * V * 4,
             lambda: oracle.shard_argmax(oracle.lm_head_logits(inp["x"], w_fp8=inp["w_fp8"], w_scale=inp["w_scale"],
                                                               max_rows_per_chunk=c["chunk"])))):
        dt_s = timed(fn)
        lm.append({"workload": 5, "weights": dt, "seconds": round(dt_s, 3), "gbs": round(nbytes / dt_s / 1e9, 2),
                   "sample": "full"})
    # workload 4: RMSNorm -> column shard, 256-row blocks for the remaining budget (at least 4 blocks)
    c = W[4]
    inp = synth.workload_inputs(4)
    x, s, w = inp["x"], inp["scale"], inp["w"]
    rows_per_block = 256
    n_blocks = x.shape[0] // rows_per_block
    left = max(1.0, budget_s - sum(t for _, _, t, _ in per) - sum(e["seconds"] for e in lm))
    done = 0
    t0 = time.perf_counter()
    while done < 4 or time.perf_counter() - t0 < left:
        r0 = (done % n_blocks) * rows_per_block
        oracle.rmsnorm_column_linear(x[r0:r0 + rows_per_block], s, w, None, [c["out_logical"]], c["tp"], c["rank"])
        done += 1
    dt4 = time.perf_counter() - t0
    rows4 = done * rows_per_block
    fl4 = 2.0 * rows4 * w.shape[0] * c["hidden"]
    full4 = 2.0 * x.shape[0] * w.shape[0] * c["hidden"]
    per.append((4, fl4, dt4, f"{rows4} rows: the 32768 rows' 256-row blocks in order, repeated past the last "
                             f"for the time budget"))
    per.sort()
    entries = [{"workload": k, "gflop": round(fl / 1e9, 3), "seconds": round(t, 3),
                "tflops": round(fl / t / 1e12, 4), "sample": smp} for k, fl, t, smp in per]
    # the headline: the step's GEMM flops over the oracle's time for them, workload 4 scaled to its 32768 rows
    step_s = sum(t for k, fl, t, _ in per if k != 4) + dt4 * full4 / fl4
    step_fl = sum(fl for k, fl, t, _ in per if k != 4) + full4
    return {
        "value": step_fl / step_s / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
        "sample": f"numpy float64 oracle on workloads 1-3 and 5 in full and {rows4} rows of workload 4 "
                  f"(the step's GEMM flops over its time, workload 4 scaled to 32768 rows: {step_s:.1f} s per step); "
                  f"{sum(t for _, _, t, _ in per) + sum(e['seconds'] for e in lm):.1f} s of oracle time "
                  f"({time.perf_counter() - t_all:.1f} s with input generation); {os.cpu_count()} host cpus, "
                  f"{_cpu_model()}",
        "per_config": entries + lm,
    }


# The dominant kernel of a step is the column GEMM of the RMSNorm workload (about 90% of the
# step's time; its normalisation pass is a separate kernel). Its launches are timed alone after
# the timed steps, with HIP events on the stream it runs on, on the normalised rows the fused
# entry point materialises: the same kernel, shape and tile as inside the step.
DOMINANT = {4: ("column GEMM [32768 x 8192] x [3072 x 8192]^T -> bf16", "gemm_nt_pair_kernel"),
            3: ("c_proj row partial [8192 x 1792] x [4096 x 1792]^T -> f32", "gemm_nt_pair_kernel"),
            2: ("fused-QKV column GEMM [4096 x 4096] x [768 x 4096]^T + bias -> bf16", "gemm_nt_dma_kernel")}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_column_32768x3072x8192_hbm_traffic.txt")
# The dominant kernel's sources: gemm.hip, common.h and the GEMM declarations of kernels.h (from
# its GemmEpilogue to launch_gemm_fp8's picker); the rest of kernels.h declares other kernels.
KERNEL_SOURCES = ("tensor_transformer_linear_amd/csrc/gemm.hip", "tensor_transformer_linear_amd/csrc/common.h",
                  "tensor_transformer_linear_amd/csrc/kernels.h")
_GEMM_DECLS = ("// Output stage of the NT GEMM", "int gemm_fp8_pick_tile(int M, int N, int K);")


def kernel_source_hash() -> str:
    import hashlib

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            data = f.read()
        if rel.endswith("kernels.h"):
            a, b = data.find(_GEMM_DECLS[0].encode()), data.find(_GEMM_DECLS[1].encode())
            if a >= 0 and b > a:
                data = data[a:b + len(_GEMM_DECLS[1])]
        h.update(data)
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter summary, or None
    when there is none or the kernel's sources changed since the counters were taken."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if "=" in line and not line.lstrip().startswith("#"):
                    k, v = line.split("=", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("source_sha256_16") != kernel_source_hash():
            return None
        return int(float(kv["hbm_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


LEG_WARMUP = 30  # untimed calls before each leg's timed ones


def roofline_leg(wl, launches, stream):
    import torch

    tt = wl.tt
    pre = None
    if 4 in wl.parts:
        # The RMSNorm pass writes the normalised rows, then the GEMM launch on them is timed:
        # the two kernels of one rmsnorm_column_linear call, as the step runs them.
        c = wl.c4
        xn = torch.empty_like(wl.x4)

        def pre():
            tt.rmsnorm_rows(wl.x4, wl.s4, c["eps"], xn, wl.ws4)

        def launch():
            tt.tp_column_linear(xn, wl.w4, None, [c["out_logical"]], c["tp"], c["rank"], y=wl.y4)
        flops, key = wl.flops[4], 4
    elif 3 in wl.parts:
        launch, flops, key = wl.part3b, wl.flops[3] / 2, 3
    elif 2 in wl.parts:
        launch, flops, key = wl.part2, wl.flops[2], 2
    else:
        return None

    def events():
        return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]

    def timed(evs, with_pre):
        for a, b in evs:
            if with_pre:
                pre()
            a.record(stream)
            launch()
            b.record(stream)

    evs, evs_b2b = events(), events()
    torch.cuda.synchronize()
    # Untimed warm-up, with no synchronize between it and the timed launches: the first
    # launches after an idle moment run up to 40% slower while the power controller settles
    # (kernel traces show it), unlike the launches inside the timed steps.
    for _ in range(LEG_WARMUP):
        if pre is not None:
            pre()
        launch()
    timed(evs, pre is not None)
    if pre is not None:
        timed(evs_b2b, False)
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3
    us_b2b = float(np.mean([a.elapsed_time(b) for a, b in evs_b2b])) * 1e3 if pre is not None else us
    ach = flops / (us * 1e-6) / 1e12
    traffic = measured_traffic() if key == 4 else None
    out = {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
           "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
           "kernel": DOMINANT[key][1], "launch": DOMINANT[key][0], "flops_per_launch": flops,
           "mean_launch_us": round(us, 2), "launches_timed": launches,
           "algorithmic_bytes_per_launch": (32768 * 8192 + 3072 * 8192 + 32768 * 3072) * 2 if key == 4 else None}
    if pre is not None:
        out["timing"] = ("HIP events around each GEMM launch, each launch right after the RMSNorm pass that "
                         "feeds it (the two kernels of the workload's call)")
        out["back_to_back_mean_launch_us"] = round(us_b2b, 2)
        out["back_to_back_frac"] = round(flops / (us_b2b * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4)
    return out


PEAK_FP8_TFLOPS = 5033.2  # MI355X dense fp8 MFMA


def fp8_prefill_leg(launches, stream):
    """The fp8 prefill column linear on the RMSNorm workload's shapes (x [32768, 8192], column
    shard [3072, 8192] quantised per output channel): per-row E4M3 quantisation of x, then the
    E4M3 x E4M3 GEMM with both scales applied in its epilogue. Each kernel is timed with HIP
    events on the stream it runs on."""
    import torch

    import synth
    import tensor_transformer_linear_amd as tt

    c = synth.WORKLOADS[4]
    inp = synth.workload_inputs(4)
    wq, ws = synth.quantize_e4m3_channels(inp["w"])
    dev = torch.device("cuda:0")
    x = torch.from_numpy(inp["x"].view(np.int16)).view(torch.bfloat16).to(dev)
    wq_d, ws_d = torch.from_numpy(wq).to(dev), torch.from_numpy(ws).to(dev)
    M, K = x.shape
    N = wq.shape[0]
    q = torch.empty((M, K), dtype=torch.uint8, device=dev)
    s = torch.empty((M,), dtype=torch.float32, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def run(ev=None):
        if ev is not None:
            ev[0].record(stream)
        tt.tp_quantize_rows_e4m3(x, q, s)
        if ev is not None:
            ev[1].record(stream)
        tt.tp_column_linear_fp8(q, s, wq_d, ws_d, None, [c["out_logical"]], c["tp"], c["rank"], y=y)
        if ev is not None:
            ev[2].record(stream)

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(launches)]
    torch.cuda.synchronize()
    for _ in range(LEG_WARMUP):  # past the power controller's settling transient, no synchronize after
        run()
    for ev in evs:
        run(ev)
    torch.cuda.synchronize()
    q_us = float(np.mean([e[0].elapsed_time(e[1]) for e in evs])) * 1e3
    g_us = float(np.mean([e[1].elapsed_time(e[2]) for e in evs])) * 1e3
    flops = 2.0 * M * N * K
    tf = flops / (g_us * 1e-6) / 1e12
    q_bytes = M * K * 3 + M * 4  # bf16 read, codes written, scales written
    return {"workload": "fp8 prefill column shard: quantise x [32768, 8192] per row to E4M3, "
                        "E4M3 GEMM with W [3072, 8192] (per-channel scales), bf16 out",
            "quantize_mean_us": round(q_us, 2), "quantize_gbs": round(q_bytes / (q_us * 1e-6) / 1e9, 1),
            "gemm_mean_us": round(g_us, 2), "gemm_tflops": round(tf, 1),
            "gemm_frac_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4), "peak_fp8_tflops": PEAK_FP8_TFLOPS,
            "end_to_end_tflops": round(flops / ((q_us + g_us) * 1e-6) / 1e12, 1), "launches_timed": launches}


def swiglu_leg(launches, stream):
    """The fused q_wi projection with its SwiGLU and the fused o_wo partial, one rank's share of a
    PaLM-style layer: 8192 tokens, E 8192, 64 heads of 128, d_ff 32768 spread over the heads
    (512 per head), tp 8 rank 0 (8 heads): q_wi W [8 x 1152, 8192], o_wo W [8192, 8 x 640].
    Each entry point is timed with HIP events on the stream it runs on."""
    import torch

    import synth
    import tensor_transformer_linear_amd as tt

    M, E, heads, padded, qkv, ff, tp, rank = 8192, 8192, 64, 0, 128, 32768, 8, 0
    h_r, fph = heads // tp, ff // (heads - padded)
    qph, fused = qkv + 2 * fph, qkv + fph
    dev = torch.device("cuda:0")

    def normal(shape, std, tid):
        return torch.from_numpy(synth.bf16_normal(shape, std, 12, tid).view(np.int16)).view(torch.bfloat16).to(dev)

    x = normal((M, E), 1.0, 0)
    w = normal((h_r * qph, E), 0.02, 1)
    w_o = normal((E, h_r * fused), 0.02, 2)
    yf = normal((M, h_r, fused), 1.0, 3)  # attention slots hold a synthetic attention output
    q = torch.empty((M, h_r, qkv), dtype=torch.bfloat16, device=dev)
    out = torch.empty((M, E), dtype=torch.float32, device=dev)

    def run(ev=None):
        if ev is not None:
            ev[0].record(stream)
        tt.tp_qwi_swiglu(x, heads, padded, qkv, ff, tp, rank, w, yf, q=q)
        if ev is not None:
            ev[1].record(stream)
        tt.tp_o_wo_partial(yf.view(M, -1), heads, padded, qkv, ff, tp, rank, w_o, out)
        if ev is not None:
            ev[2].record(stream)

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(launches)]
    torch.cuda.synchronize()
    for _ in range(LEG_WARMUP):  # past the power controller's settling transient, no synchronize after
        run()
    for ev in evs:
        run(ev)
    torch.cuda.synchronize()
    a_us = float(np.mean([e[0].elapsed_time(e[1]) for e in evs])) * 1e3
    o_us = float(np.mean([e[1].elapsed_time(e[2]) for e in evs])) * 1e3
    a_fl = 2.0 * M * E * h_r * qph
    o_fl = 2.0 * M * E * h_r * fused
    a_tf, o_tf = a_fl / (a_us * 1e-6) / 1e12, o_fl / (o_us * 1e-6) / 1e12
    return {"workload": "fused q_wi + SwiGLU and o_wo, 8192 tokens, E 8192, 64 heads x 128, d_ff 32768, tp 8 rank 0",
            "qwi_swiglu_mean_us": round(a_us, 2), "qwi_swiglu_tflops": round(a_tf, 1),
            "qwi_swiglu_frac_bf16_peak": round(a_tf / PEAK_BF16_TFLOPS, 4),
            "o_wo_mean_us": round(o_us, 2), "o_wo_tflops": round(o_tf, 1),
            "o_wo_frac_bf16_peak": round(o_tf / PEAK_BF16_TFLOPS, 4),
            "layer_tflops": round((a_fl + o_fl) / ((a_us + o_us) * 1e-6) / 1e12, 1), "launches_timed": launches}


def reduce_scatter_leg(launches, stream):
    """The sequence-parallel reduce-scatter of the c_proj partials with the residual add, for the
    llama-8B MLP shard (batch 8, seq 1024, hidden 4096, tp 8): the eight ranks' float32 partials
    [8192, 4096] summed in rank order over each destination's 1024-row slice, plus a bf16 residual,
    bf16 out. One launch per destination rank. A launch takes about 25 us, less than the binding's
    host work per call, so eagerly issued calls leave the GPU waiting between launches: the eight
    launches are captured once in a HIP graph and replayed, with HIP events around each replay."""
    import torch

    import synth
    import tensor_transformer_linear_amd as tt

    batch, seq, tp, N = 8, 1024, 8, 4096
    M, rows = batch * seq, batch * seq // tp
    dev = torch.device("cuda:0")
    parts = [torch.from_numpy(synth.rng(13, r).standard_normal((M, N), dtype=np.float32)).to(dev) for r in range(tp)]
    res = [torch.from_numpy(synth.bf16_normal((rows, N), 1.0, 13, 100 + d).view(np.int16)).view(torch.bfloat16).to(dev)
           for d in range(tp)]
    z = torch.empty((rows, N), dtype=torch.bfloat16, device=dev)

    def all_ranks():
        for d in range(tp):
            tt.tp_reduce_scatter_residual(parts, batch, seq, d, residual=res[d], z=z)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        all_ranks()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        all_ranks()
    graph.replay()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record(stream)
        graph.replay()
        b.record(stream)
    torch.cuda.synchronize()
    t = [a.elapsed_time(b) * 1e3 / tp for a, b in evs]  # per launch
    us = float(np.median(t))
    nbytes = tp * rows * N * 4 + rows * N * 2 + rows * N * 2  # partial slices, residual, z
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": "sequence-parallel reduce-scatter + residual, llama-8B MLP shard: 8 partials [8192, 4096] f32, "
                        "tp 8, one destination rank per launch",
            "median_us": round(us, 2), "mean_us": round(float(np.mean(t)), 2), "bytes_per_launch": nbytes,
            "gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4), "launches_timed": launches * tp,
            "timing": "a HIP graph of the eight destination launches, replayed with HIP events around each "
                      "replay; per launch = replay time / 8; throughput from the median"}


def embedding_leg(launches, stream):
    """The vocab-parallel embedding (one rank's share) at the RMSNorm workload's prefill size:
    32768 token ids uniform over a 128256-token vocabulary, tp 8 rank 0 (16032 table rows of
    8192 bf16), so one token in eight reads a table row and every token writes an output row."""
    import torch

    import synth
    import tensor_transformer_linear_amd as tt

    vocab, tp, rank, E, n = 128256, 8, 0, 8192, 16 * 2048
    rows = vocab // tp
    dev = torch.device("cuda:0")
    tbl = torch.from_numpy(synth.bf16_normal((rows, E), 1.0, 6, 1).view(np.int16)).view(torch.bfloat16).to(dev)
    tok = torch.from_numpy(synth.rng(6, 0).integers(0, vocab, n).astype(np.int32)).to(dev)
    out = torch.empty((n, E), dtype=torch.bfloat16, device=dev)
    hits = int(((tok >= 0) & (tok < rows)).sum().item())
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
    torch.cuda.synchronize()
    for _ in range(LEG_WARMUP):  # no synchronize between the warm-up and the timed launches
        tt.tp_vocab_embedding(tok, vocab, tp, rank, tbl, out)
    for a, b in evs:
        a.record(stream)
        tt.tp_vocab_embedding(tok, vocab, tp, rank, tbl, out)
        b.record(stream)
    torch.cuda.synchronize()
    t = [a.elapsed_time(b) * 1e3 for a, b in evs]
    us = float(np.median(t))
    nbytes = hits * E * 2 + n * 4 + n * E * 2
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": "vocab-parallel embedding, 32768 tokens, E 8192, vocab 128256, tp 8 rank 0",
            "median_us": round(us, 2), "mean_us": round(float(np.mean(t)), 2), "bytes": nbytes, "gbs": round(gbs, 1),
            "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4), "rows_read": hits, "launches_timed": launches,
            "timing": "per-launch HIP events; throughput from the median"}


def gemm_launches(n: int) -> None:
    """Each GEMM launch of the hot path, n times in a row, in a fixed order (a profiler's dispatch
    list then reads in that order); the labels go to stderr."""
    import torch

    import synth
    import tensor_transformer_linear_amd as tt

    dev = torch.device("cuda:0")
    wl = Workloads({1, 2, 3, 4}, dev)
    c4 = wl.c4
    xn = torch.empty_like(wl.x4)
    tt.rmsnorm_column_linear(wl.x4, wl.s4, c4["eps"], wl.w4, None, [c4["out_logical"]], c4["tp"], c4["rank"], y=wl.y4,
                             workspace=wl.ws4, xnorm_out=xn)
    c1 = wl.c1
    segs = [
        ("workload 1 c_fc + GELU, both ranks [256 x 768] x [1536 x 768]^T",
         lambda: [tt.tp_column_linear(wl.x1, wl.wfc1[r], None, [c1["inter"]], c1["tp"], r, act=tt.TP_ACT_GELU_ERF,
                                      y=wl.g1[r]) for r in range(2)]),
        ("workload 1 c_proj partials, both ranks [256 x 1536] x [768 x 1536]^T",
         lambda: [tt.tp_row_linear_partial(wl.g1[r], c1["inter"], wl.wpj1[r], None, c1["tp"], r, y_partial=wl.s1,
                                           accumulate=int(r > 0)) for r in range(2)]),
        ("workload 2 fused QKV [4096 x 4096] x [768 x 4096]^T + bias", wl.part2),
        ("workload 3 c_fc + GELU [8192 x 4096] x [1792 x 4096]^T", wl.part3a),
        ("workload 3 c_proj partial [8192 x 1792] x [4096 x 1792]^T", wl.part3b),
        ("workload 4 column GEMM [32768 x 8192] x [3072 x 8192]^T",
         lambda: tt.tp_column_linear(xn, wl.w4, None, [c4["out_logical"]], c4["tp"], c4["rank"], y=wl.y4)),
    ]
    inp = synth.workload_inputs(4)
    wq, ws = synth.quantize_e4m3_channels(inp["w"])
    wq_d, ws_d = torch.from_numpy(wq).to(dev), torch.from_numpy(ws).to(dev)
    q, sc = tt.tp_quantize_rows_e4m3(wl.x4)
    segs.append(("fp8 prefill GEMM [32768 x 8192] x [3072 x 8192]^T (E4M3)",
                 lambda: tt.tp_column_linear_fp8(q, sc, wq_d, ws_d, None, [c4["out_logical"]], c4["tp"], c4["rank"],
                                                 y=wl.y4)))
    M, E, heads, qkv, ff, tp = 8192, 8192, 64, 128, 32768, 8
    h_r, fph = heads // tp, ff // heads

    def normal(shape, std, tid):
        return torch.from_numpy(synth.bf16_normal(shape, std, 12, tid).view(np.int16)).view(torch.bfloat16).to(dev)
    xq = normal((M, E), 1.0, 0)
    wqwi = normal((h_r * (qkv + 2 * fph), E), 0.02, 1)
    w_o = normal((E, h_r * (qkv + fph)), 0.02, 2)
    yf = normal((M, h_r, qkv + fph), 1.0, 3)
    qq = torch.empty((M, h_r, qkv), dtype=torch.bfloat16, device=dev)
    out = torch.empty((M, E), dtype=torch.float32, device=dev)
    segs.append(("q_wi: SwiGLU columns then query columns, E 8192, 8 heads x (128 + 2 x 512)",
                 lambda: tt.tp_qwi_swiglu(xq, heads, 0, qkv, ff, tp, 0, wqwi, yf, q=qq)))
    segs.append(("o_wo partial [8192 x 5120] x [8192 x 5120]^T",
                 lambda: tt.tp_o_wo_partial(yf.view(M, -1), heads, 0, qkv, ff, tp, 0, w_o, out)))
    torch.cuda.synchronize()
    for label, fn in segs:
        print(f"gemm-launches: {n} x {label}", file=sys.stderr, flush=True)
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
    print(json.dumps({"gemm_launches": n, "segments": [l for l, _ in segs]}), flush=True)


def lm_shapes(shapes) -> None:
    """The decode LM head under each given launch shape: 32 and 64 batch rows, bf16 and E4M3
    weights rotating over >= 512 MB of copies, 5 + 20 calls per setting, event-timed (the call
    times include the host's launch work; the kernels' own times come from a kernel trace)."""
    import torch

    import synth
    import tensor_transformer_linear_amd as tt

    dev = torch.device("cuda:0")
    c = synth.WORKLOADS[5]
    inp = synth.workload_inputs(5)
    w = torch.from_numpy(inp["w"].view(np.int16)).view(torch.bfloat16).to(dev)
    q, sc = torch.from_numpy(inp["w_fp8"]).to(dev), torch.from_numpy(inp["w_scale"]).to(dev)
    w16 = [w] + [w.clone() for _ in range(max(1, -(-(512 << 20) // (w.numel() * 2)) - 1))]
    w8 = [(q, sc)] + [(q.clone(), sc.clone()) for _ in range(max(1, -(-(512 << 20) // q.numel()) - 1))]
    out = []
    for B in (32, 64):
        x = torch.from_numpy(synth.bf16_normal((B, w.shape[1]), 1.0, 5, 77).view(np.int16)).view(torch.bfloat16).to(dev)
        ws = tt.lm_head_workspace(B, c["vocab"], c["tp"], c["rank"], dev)
        for shape in shapes:
            for fp8 in (False, True):
                print(f"lm-shapes: B {B} shape {shape} {'fp8' if fp8 else 'bf16'}", file=sys.stderr, flush=True)

                def call(i):
                    if fp8:
                        qq, ss = w8[i % len(w8)]
                        tt.lm_head_shard_argmax(x, c["vocab"], c["tp"], c["rank"], c["chunk"], qq,
                                                tt.TP_DTYPE_FP8_E4M3, ss, workspace=ws)
                    else:
                        tt.lm_head_shard_argmax(x, c["vocab"], c["tp"], c["rank"], c["chunk"], w16[i % len(w16)],
                                                workspace=ws)
                with tt.tuning(lm_shape=shape):
                    for i in range(5):
                        call(i)
                    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                          for _ in range(20)]
                    torch.cuda.synchronize()
                    for i, (a, b) in enumerate(ev):
                        a.record()
                        call(i)
                        b.record()
                    torch.cuda.synchronize()
                t = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
                out.append({"batch_rows": B, "shape": shape, "weights": "fp8" if fp8 else "bf16",
                            "call_median_us": round(t[10], 2)})
    print(json.dumps({"lm_shapes": out}), flush=True)


def stream_probe(n: int) -> None:
    """The tuning library's fetch-shape probe over a bf16 LM-head weight shard (16032 rows x
    8192 bytes) rotating over five copies: n launches per shape, HIP events per launch."""
    import torch

    import tensor_transformer_linear_amd as tt

    rows, rowb = 16032, 8192
    copies = [torch.full((rows * rowb,), 17, dtype=torch.uint8, device="cuda") for _ in range(5)]
    out = torch.zeros(rows // 64 + 1, dtype=torch.int32, device="cuda")
    T = tt.tuning_lib()
    stream = torch.cuda.current_stream()
    names = ["16 rows x 64 B", "8 rows x 128 B", "4 rows x 256 B", "1 row x 1 KB, rows interleaved",
             "1 row x 1 KB, each wave's rows in order", "each 64-row block in order",
             "4 rows x 256 B in the row-quad kernel's window order",
             "4 rows x 256 B in the row-quad kernel's window order, staggered slices"]
    res = []
    for shape, nt in [(s, 1) for s in range(8)] + [(0, 0), (5, 0)]:
        print(f"stream-probe: shape {shape} nontemporal {nt}", file=sys.stderr, flush=True)
        t = []
        for i in range(n + 3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            st = T.tpt_stream_probe(shape, nt, copies[i % 5].data_ptr(), rows, out.data_ptr(),
                                    ctypes.c_void_p(stream.cuda_stream))
            b.record(stream)
            if st != 0:
                raise RuntimeError(f"tpt_stream_probe returned {st}")
            b.synchronize()
            if i >= 3:
                t.append(a.elapsed_time(b) * 1e3)
        t.sort()
        med = t[len(t) // 2]
        res.append({"shape": shape, "fetch": names[shape], "nontemporal": nt, "median_us": round(med, 2),
                    "min_us": round(t[0], 2), "gbs": round(rows * rowb / med / 1e3, 1)})
    print(json.dumps({"stream_probe": res, "bytes": rows * rowb, "launches": n}), flush=True)


def mfma_rate(seconds: float, wgs: int, fp8: int) -> None:
    """The matrix rate the chip sustains: the tuning library's probe (``wgs`` workgroups of 4
    waves, each wave 4 independent v_mfma_f32_32x32x16_bf16 chains, or with ``fp8``
    v_mfma_scale_f32_32x32x64_f8f6f4 chains, on pseudo-random operands; 4000 rounds, 2000 for
    E4M3: 2.15 or 4.29 TFLOP per launch at 1024 workgroups) back to back for about ``seconds``,
    HIP events per launch."""
    import torch

    import tensor_transformer_linear_amd as tt

    iters = 2000 if fp8 else 4000
    flops = wgs * 4 * iters * 4 * 32 * 32 * (64 if fp8 else 16) * 2
    out = torch.zeros(wgs, dtype=torch.float32, device="cuda")
    T = tt.tuning_lib()
    stream = torch.cuda.current_stream()
    h = ctypes.c_void_p(stream.cuda_stream)
    t_ms = []
    t0 = time.perf_counter()
    last = t0
    while time.perf_counter() - t0 < seconds:
        batch = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(50)]
        for a, b in batch:
            a.record(stream)
            if T.tpt_mfma_rate(fp8, wgs, iters, out.data_ptr(), h) != 0:
                raise RuntimeError("tpt_mfma_rate failed")
            b.record(stream)
        torch.cuda.synchronize()
        t_ms += [a.elapsed_time(b) for a, b in batch]
        if time.perf_counter() - last > 1.0:
            last = time.perf_counter()
            print(f"mfma-rate: {len(t_ms)} launches, last {flops / t_ms[-1] / 1e9:.0f} TFLOP/s", file=sys.stderr,
                  flush=True)
    tf = [flops / t / 1e9 for t in t_ms]
    tail = sorted(tf[len(tf) * 4 // 5:])
    print(json.dumps({"mfma_rate": {"instruction": "v_mfma_scale_f32_32x32x64_f8f6f4" if fp8 else "v_mfma_f32_32x32x16_bf16",
                                    "workgroups": wgs, "waves_per_simd": wgs * 4 // 1024, "flops_per_launch": flops,
                                    "launches": len(tf), "seconds": round(sum(t_ms) / 1e3, 2),
                                    "first_5_median_tflops": round(float(np.median(tf[:5])), 1),
                                    "last_fifth_median_tflops": round(tail[len(tail) // 2], 1),
                                    "max_tflops": round(max(tf), 1),
                                    "peak_tflops": PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS}}),
          flush=True)


def copy_probe(mb: int):
    """Plain device-to-device copies of a known size: the reference for HBM byte counters."""
    import torch

    n = mb << 20
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "launches": 3}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the library computes tensor-parallel ranks shard by shard on a "
              f"single device and has no multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import torch

    import tensor_transformer_linear_amd as tt

    tt.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_probe > 0:
        copy_probe(args.copy_probe)
        return
    if args.gemm_launches > 0:
        gemm_launches(args.gemm_launches)
        return
    if args.lm_shapes:
        lm_shapes([int(v) for v in args.lm_shapes.split(",") if v])
        return
    if args.stream_probe > 0:
        stream_probe(args.stream_probe)
        return
    if args.mfma_rate > 0:
        mfma_rate(args.mfma_rate, args.mfma_rate_workgroups, args.mfma_rate_fp8)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    parts = {int(p) for p in args.parts.split(",") if p}
    t_setup = time.perf_counter()
    wl = Workloads(parts, dev)
    torch.cuda.synchronize()
    print(f"bench: inputs ready in {time.perf_counter() - t_setup:.1f} s", file=sys.stderr, flush=True)

    segs = wl.segments()
    stream = torch.cuda.current_stream()

    def step(evs=None):
        for i, (_, fn) in enumerate(segs):
            if evs is not None:
                evs[i][0].record(stream)
            fn()
            if evs is not None:
                evs[i][1].record(stream)
        if 5 in parts:
            wl.rot += 1

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in segs]
              for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for k in range(args.steps):
        step(events[k])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    per_seg = {name: [events[k][i][0].elapsed_time(events[k][i][1]) for k in range(args.steps)]
               for i, (name, _) in enumerate(segs)}
    avg = {n: float(np.mean(v)) for n, v in per_seg.items()}
    med = {n: float(np.median(v)) for n, v in per_seg.items()}
    print("bench: per-part mean ms " + json.dumps({n: round(v, 4) for n, v in avg.items()}), file=sys.stderr,
          flush=True)

    gemm_names = {1: ["gpt2_mlp_tp2_both_ranks"], 2: ["qkv_gqa_column"],
                  3: ["llama8b_c_fc_gelu", "llama8b_c_proj_partial"], 4: ["rmsnorm_column"]}
    per_config = []
    gemm_flops = gemm_ms = 0.0
    for cfg in (1, 2, 3, 4):
        if cfg not in parts:
            continue
        ms = sum(avg[n] for n in gemm_names[cfg])
        tf = wl.flops[cfg] / (ms * 1e-3) / 1e12
        gemm_flops += wl.flops[cfg]
        gemm_ms += ms
        per_config.append({"workload": cfg, "parts": gemm_names[cfg], "mean_us": round(ms * 1e3, 2),
                           "median_us": round(sum(med[n] for n in gemm_names[cfg]) * 1e3, 2),
                           "gflop": round(wl.flops[cfg] / 1e9, 3), "tflops": round(tf, 1),
                           "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)})
        if cfg == 3:
            for n, fl in (("llama8b_c_fc_gelu", wl.flops[3] / 2), ("llama8b_c_proj_partial", wl.flops[3] / 2)):
                per_config[-1][n + "_tflops"] = round(fl / (avg[n] * 1e-3) / 1e12, 1)
    lm = {}
    if 5 in parts:
        for dt in ("bf16", "fp8"):
            ms = avg[f"lm_head_{dt}"]
            gbs = wl.bytes5[dt] / (ms * 1e-3) / 1e9
            lm[dt] = {"mean_us": round(ms * 1e3, 2), "median_us": round(med[f"lm_head_{dt}"] * 1e3, 2),
                      "bytes": wl.bytes5[dt], "gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
            per_config.append({"workload": 5, "weights": dt, **lm[dt]})

    value = gemm_flops / (gemm_ms * 1e-3) / 1e12 if gemm_ms > 0 else None
    roofline = roofline_leg(wl, args.steps, stream) if gemm_ms > 0 else None
    fp8 = fp8_prefill_leg(args.steps, stream) if args.next else None
    glu = swiglu_leg(args.steps, stream) if args.next else None
    emb = embedding_leg(args.steps, stream) if args.next else None
    rsc = reduce_scatter_leg(args.steps, stream) if args.next else None
    out = {
        "metric": METRIC, "value": round(value, 2) if value else None, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) activations and N(0,0.02) random-init weights of the workloads' shapes",
        "config": {"workload": "one pass of: gpt2-small MLP tp2 (both ranks), fused-QKV GQA column tp8 r0, "
                               "llama-8B MLP tp8, RMSNorm->column [32768x8192]x[3072], decode LM head vocab 128256 "
                               "tp8 r0 (bf16 and e4m3 weights)",
                   "gemm_flops_per_step": gemm_flops, "gemm_ms_per_step": round(gemm_ms, 4),
                   "parts": sorted(parts)},
        "roofline": roofline,
        "lm_head": lm or None,
        "fp8_prefill": fp8,
        "swiglu": glu,
        "embedding": emb,
        "reduce_scatter": rsc,
        "per_config": per_config,
    }
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
