"""Build ``libtpshard.so`` (the gfx950 HIP kernels and their C ABI) in-tree with hipcc.

The same objects, plus the launch-choice entry points of ``csrc/tuning_abi.hip``, also link
``libtpshard_tuning.so``, which the tests and measurements use to force a tile, a main loop or
an LM-head launch shape. The product library does not contain those entry points."""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtpshard.so")
TUNING_LIB = os.path.join(PKG, "libtpshard_tuning.so")
SOURCES = ["tpshard_abi.hip", "gemm.hip", "rmsnorm.hip", "lm_head.hip", "quant.hip", "embed.hip", "reduce.hip"]
TUNING_SOURCES = ["tuning_abi.hip", "probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libtpshard")


def flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        # no packed float32 instructions anywhere in the device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    ]


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every HIP source for gfx950 and link both shared libraries; returns the product
    library's path."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()

    def compile_one(src: str) -> str:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        if verbose:
            print(" ".join(cmd))
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES + TUNING_SOURCES))
    n = len(SOURCES)
    for out, parts in ((LIB, objs[:n]), (TUNING_LIB, objs)):
        tmp = out + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *parts, "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link of {os.path.basename(out)} failed:\n{r.stderr}")
        os.replace(tmp, out)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
