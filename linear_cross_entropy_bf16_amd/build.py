"""Build libflce.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m linear_cross_entropy_bf16_amd.build [--if-stale] [--jobs N]

The kernels are compiled as several object files in parallel (one per
element type and option key of the large GEMM kernels, see csrc/flce_launch.hpp)
and linked into one shared library written next to this file, so it travels
with the source tree.  Packed fp32 instructions are disabled for all device
code.  Every object depends on every file under csrc/ and include/, so any
source edit rebuilds the whole library.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ_DIR = os.path.join(HERE, "_build")
LIB_NAME = "libflce.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = "gfx950"

FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

ELEM_TYPES = {"bf16": "uint16_t", "f32": "float"}


def units():
    """(object name, source, defines) of every object file of the library."""
    out = [("flce", "flce.hip", {})]
    for tag, t in ELEM_TYPES.items():
        for key in range(8):
            out.append((f"fwd_{tag}_{key}", "flce_fwd.hip", {"FLCE_T": t, "FLCE_KEY": key}))
            out.append((f"g_{tag}_{key}", "flce_bwd.hip", {"FLCE_T": t, "FLCE_KEY": key}))
        out.append((f"dwdx_{tag}", "flce_bwd.hip", {"FLCE_T": t}))
        out.append((f"ce_{tag}", "flce_ce.hip", {"FLCE_T": t}))
    return out


def depends() -> list:
    """Every file whose edit must rebuild the library."""
    files = sorted(glob.glob(os.path.join(CSRC, "*")))
    files += sorted(glob.glob(os.path.join(INCLUDE, "*.h")))
    files.append(os.path.abspath(__file__))
    return files


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libflce.so")


def compile_command(src: str, obj: str, defines: dict) -> list:
    defs = [f"-D{k}={v}" for k, v in defines.items()]
    return [hipcc(), *FLAGS, *defs, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]


def link_command(objs: list, out: str) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out]


def up_to_date() -> bool:
    if not os.path.exists(LIB_PATH):
        return False
    t = os.path.getmtime(LIB_PATH)
    return all(os.path.getmtime(p) <= t for p in depends())


def _run(cmd: list, verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}: {' '.join(cmd)}")


def build(force: bool = True, verbose: bool = True, jobs: int = 0) -> str:
    """Compile libflce.so; with force=False only when a source is newer."""
    if not force and up_to_date():
        return LIB_PATH
    os.makedirs(OBJ_DIR, exist_ok=True)
    jobs = jobs or min(16, os.cpu_count() or 1)
    work = [(compile_command(src, os.path.join(OBJ_DIR, name + ".o"), defs), os.path.join(OBJ_DIR, name + ".o"))
            for name, src, defs in units()]
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        for f in [pool.submit(_run, cmd, verbose) for cmd, _ in work]:
            f.result()
    tmp = LIB_PATH + ".tmp"
    _run(link_command([obj for _, obj in work], tmp), verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    jobs = 0
    if "--jobs" in sys.argv:
        jobs = int(sys.argv[sys.argv.index("--jobs") + 1])
    build(force="--if-stale" not in sys.argv, jobs=jobs)
