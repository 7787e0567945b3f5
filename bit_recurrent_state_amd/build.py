"""Compile libqstate.so (gfx950) in-tree with hipcc.

Each kernel source (one per dk and scale-group axis) and the host sources
compile to objects in parallel under _build/, then link into the shared
library.  Flags: no FP contraction (every fused multiply-add in the kernels
is an explicit fmaf), IEEE-correct FP32 division, FP32 denormals kept,
and packed FP32 instructions switched off.
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libqstate.so")
SOURCES = ([os.path.join(CSRC, f"qstate_window_dk{dk}_w{w}.hip")
            for dk in (64, 128, 256) for w in (4, 8, 16)]
           + [os.path.join(CSRC, f"qstate_{kind}_dk{dk}.hip")
              for kind in ("value", "key") for dk in (64, 128, 256)]
           + [os.path.join(CSRC, "qstate_ceiling.hip")]
           + [os.path.join(CSRC, "qstate_dispatch.cpp"), os.path.join(CSRC, "qstate_api.cpp")])
HEADERS = [os.path.join(ROOT, "include", h) for h in ("qstate.h", "qstate_ceiling.h")] + [
    os.path.join(CSRC, h) for h in ("qstate_launch.h", "qstate_device.h", "qstate_value.h",
                                    "qstate_key.h", "qstate_window.h",
                                    "qstate_persist.h")]
BUILD = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def compile_command(src: str, obj: str, extra=()) -> list:
    return [HIPCC, *FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c",
            "-o", obj, src]


def build(out: str = LIB, extra=(), jobs: int = 0) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1, 16)
    objs = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in SOURCES]
    pending = list(zip(SOURCES, objs))
    running = []
    failed = []
    while pending or running:
        while pending and len(running) < jobs:
            src, obj = pending.pop(0)
            running.append((src, subprocess.Popen(compile_command(src, obj, extra))))
        src, proc = running.pop(0)
        if proc.wait() != 0:
            failed.append(src)
    if failed:
        raise subprocess.CalledProcessError(1, f"hipcc: {', '.join(failed)}")
    digest = source_hash()
    tmp = out + ".tmp"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs],
                   check=True)
    os.replace(tmp, out)
    if out == LIB:
        with open(HASH_FILE, "w") as fh:
            fh.write(digest + "\n")
    return out


HASH_FILE = LIB + ".srchash"


def source_hash() -> str:
    """sha256[:16] of every source and header the library is built from and
    of the compile flags: a built library records it, and a library whose
    record differs from the sources at hand is stale."""
    import hashlib
    h = hashlib.sha256()
    for f in sorted(SOURCES + HEADERS):
        h.update(os.path.basename(f).encode() + b"\0")
        with open(f, "rb") as fh:
            h.update(fh.read())
    h.update("\0".join(FLAGS).encode())
    return h.hexdigest()[:16]


def unit_hash(unit: str) -> str:
    """sha256[:16] of one kernel translation unit (a file name in csrc/), every
    header it includes, directly or not, the host code that configures its
    launches, and the compile flags: profiler counts taken on a kernel stay
    valid while this hash does, whatever else in the library changes."""
    import hashlib
    import re
    dirs = [CSRC, os.path.join(ROOT, "include")]
    seen, todo = [], [unit, "qstate_dispatch.cpp", "qstate_api.cpp"]
    while todo:
        name = todo.pop()
        if name in seen:
            continue
        path = next((os.path.join(d, name) for d in dirs if os.path.exists(os.path.join(d, name))),
                    None)
        if path is None:
            continue
        seen.append(name)
        with open(path, "rb") as fh:
            text = fh.read()
        todo += [m.decode() for m in re.findall(rb'#include "([^"]+)"', text)]
    h = hashlib.sha256()
    for name in sorted(seen):
        path = next(os.path.join(d, name) for d in dirs if os.path.exists(os.path.join(d, name)))
        h.update(name.encode() + b"\0")
        with open(path, "rb") as fh:
            h.update(fh.read())
    h.update("\0".join(FLAGS).encode())
    return h.hexdigest()[:16]


def stale() -> bool:
    """True when the library is missing or was built from other sources or flags."""
    if not os.path.exists(LIB) or not os.path.exists(HASH_FILE):
        return True
    with open(HASH_FILE) as fh:
        return fh.read().strip() != source_hash()


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
