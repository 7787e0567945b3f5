"""Compile libqstate.so (gfx950) in-tree with hipcc.

Flags: no FP contraction (every fused multiply-add in the kernels is an
explicit fmaf), IEEE-correct FP32 division, FP32 denormals kept, and packed
FP32 instructions switched off.
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libqstate.so")
SOURCES = [os.path.join(CSRC, "qstate_kernels.hip"), os.path.join(CSRC, "qstate_api.cpp")]
HEADERS = [os.path.join(ROOT, "include", "qstate.h"), os.path.join(CSRC, "qstate_launch.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def command(out: str = LIB, extra=()) -> list:
    return [HIPCC, *FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", out,
            *SOURCES]


def build(out: str = LIB, extra=()) -> str:
    tmp = out + ".tmp"
    subprocess.run(command(tmp, extra), check=True)
    os.replace(tmp, out)
    return out


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(f) > t for f in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
