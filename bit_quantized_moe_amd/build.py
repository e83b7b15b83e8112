"""Builds libbqm.so (the HIP library behind include/bqm.h) in-tree for gfx950.

python -m bit_quantized_moe_amd.build      # or build() from Python
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libbqm.so")

SOURCES = ["api.hip", "quant.hip", "route.hip", "moe.hip"]
# Bit-exact number-format code: no contraction of a*b+c into fma.
NO_CONTRACT = {"quant.hip", "route.hip", "api.hip"}

COMMON_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-I" + INCLUDE,
    "-I" + CSRC,
    # packed FP32 instructions are disabled for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wno-unused-result",
]


def _hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libbqm.so")


def _compile(src: str, objdir: str) -> str:
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    flags = list(COMMON_FLAGS)
    flags.append("-ffp-contract=off" if src in NO_CONTRACT else "-ffp-contract=fast")
    if src == "moe.hip":
        # the GEMM epilogues index 256 accumulator registers with constant indices only
        # after their loops are fully unrolled; the default limit for an unroll pragma
        # leaves the largest (SwiGLU backward) rolled and the accumulator in scratch
        flags += ["-mllvm", "-pragma-unroll-threshold=200000"]
    cmd = [_hipcc(), *flags, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-6000:]}")
    return obj


def build(verbose: bool = True) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with ThreadPoolExecutor(max_workers=min(4, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, objdir), srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-4000:]}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
