"""Builds libmeo.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc.

    python -m memory_efficient_optimizers_amd.build [--verbose]

Every source is compiled to an object in parallel, then linked into
``memory_efficient_optimizers_amd/libmeo.so``. Packed fp32 instructions are
disabled for the device code (scalar/float2 arithmetic only).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmeo.so")
SOURCES = ["abi.cpp", "passes.hip", "adafactor.hip", "came.hip", "lamb.hip", "shard.hip", "galore.hip", "galore_refresh.hip"]
ARCH = os.environ.get("MEO_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Only the fused multiply-adds written as fmaf: every compiled variant of a
    # kernel then rounds the same way, so results do not depend on the list.
    "-ffp-contract=off",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libmeo.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout or "") + (r.stderr or "")
    # The host pass does not know the device-only target feature; that warning is noise.
    lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines))


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.rsplit(".", 1)[0] + ".o")
        objs.append(obj)
        cmds.append([hipcc, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(cmds), 8)) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
