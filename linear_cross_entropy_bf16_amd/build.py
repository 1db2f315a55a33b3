"""Build libflce.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m linear_cross_entropy_bf16_amd.build

Compiles with hipcc; the library is written next to this file so it travels
with the source tree.  Packed fp32 instructions are disabled for all device
code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libflce.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = "gfx950"

SOURCES = [os.path.join(CSRC, "flce.hip")]
DEPENDS = SOURCES + [os.path.join(CSRC, f) for f in ("flce_gemm.hpp", "flce_kernels.hpp")] + [
    os.path.join(INCLUDE, "flce.h")]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libflce.so")


def command(out: str = LIB_PATH, extra=()) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC, *SOURCES, "-o", out, *extra]


def up_to_date() -> bool:
    if not os.path.exists(LIB_PATH):
        return False
    t = os.path.getmtime(LIB_PATH)
    return all(os.path.getmtime(p) <= t for p in DEPENDS)


def build(force: bool = True, verbose: bool = True) -> str:
    """Compile libflce.so; with force=False only when a source is newer."""
    if not force and up_to_date():
        return LIB_PATH
    tmp = LIB_PATH + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(force="--if-stale" not in sys.argv)
