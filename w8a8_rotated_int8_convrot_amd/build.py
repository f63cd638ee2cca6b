"""Build ``libconvrot.so`` in-tree with hipcc for gfx950.

Usage: ``python -m w8a8_rotated_int8_convrot_amd.build`` (or ``build()``).
The library is placed next to this file, where ``binding`` looks for it.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libconvrot.so")
SOURCES = ("convrot_api.hip", "rotate_quant.hip", "gemm_i8.hip", "default_path.hip", "mfma_probe.hip")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # every float operation is one IEEE operation in the written order: the
    # rotation must reproduce the same sums bit for bit, and fused multiply-adds
    # are written out explicitly where wanted
    "-ffp-contract=off",
    # fp32 '/' is the correctly rounded IEEE division
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # no packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep small per-thread arrays (staging pointers) in registers instead of
    # letting the compiler move them into LDS, which the GEMM tiles fill
    "-mllvm", "-disable-promote-alloca-to-lds",
    "-Wall",
]


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
