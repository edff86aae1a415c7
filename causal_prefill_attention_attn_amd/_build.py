"""Compile the HIP sources of the package into libcpattn.so (gfx950 only).

hipcc cross-compiles for gfx950 without a GPU present, so this runs on any
machine with ROCm installed.  The library is built in-tree, next to this
file, and loaded from there by the binding.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libcpattn.so")
SOURCES = ["attn_api.hip", "attn_bf16.hip", "attn_fp8.hip", "quant.hip", "hadamard.hip", "decode.hip"]
HEADERS = ["attn_device.h", "attn_kernels.h"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 ALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # scores and probabilities are never NaN for finite inputs; without this
    # every fmaxf over matrix-core results gets a NaN-quieting instruction
    "-fno-honor-nans",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False) -> str:
    """Always recompiles (the caller asked for a build); returns the .so path."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-I", CSRC, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libcpattn.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
