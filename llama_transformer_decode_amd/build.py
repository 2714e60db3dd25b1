"""Build libl2d.so (the HIP decode library) in-tree with hipcc for gfx950.

Every source compiles for --offload-arch=gfx950 only. Packed-fp32 VALU ops
are switched off for all device code (-packed-fp32-ops); fast-math is not
used, so fp32 division and rounding stay IEEE (the Q8_0 quantiser relies on
a correctly rounded division).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libl2d.so")

SOURCES = ["gemv.hip", "chain.hip", "attn.hip", "step.hip", "stream.hip", "prefill.hip", "gemv_noalloc.hip", "ctx.cpp", "blob.cpp", "stream_check.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
    "-Wall",
    "-Wno-unused-result",
]


# Per-source extra flags. The matvec kernel holds its input vector in arrays
# of float4 across the weight prefetch; with two or more chunks per thread
# (hidden sizes above 4096) LLVM's SROA leaves those arrays on the stack.
# The AMDGPU alloca-to-vector promotion, given a larger budget, moves them
# back into registers.
EXTRA = {
    "gemv.hip": ["-mllvm", "-amdgpu-promote-alloca-to-vector-limit=1024",
                 "-mllvm", "-amdgpu-promote-alloca-to-vector-max-regs=64"],
    "chain.hip": ["-mllvm", "-amdgpu-promote-alloca-to-vector-limit=1024",
                  "-mllvm", "-amdgpu-promote-alloca-to-vector-max-regs=64"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + CFLAGS + EXTRA.get(src, [])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every source and link libl2d.so; always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
