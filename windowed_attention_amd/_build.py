"""Compile the R-SWA HIP library (librswa.so) for gfx950, in-tree.

HIP sources are compiled with hipcc for gfx950 only; the pure C++ planning code with g++.
Packed-fp32 instructions are disabled for all device code (hipcc would otherwise form
v_pk_* float32 operations from scalar code).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "librswa.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-std=c++17", "-O3", "-fPIC", "-I", INCLUDE, "-I", CSRC]
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
HIP_SOURCES = ["rswa_api.hip", "append.hip", "decode.hip", "prefill.hip", "prefill_bwd.hip"]
CXX_SOURCES = ["plan.cpp"]
# Per-source extra flags. The prefill kernel produces no NaN (masked scores are -inf, never
# inf - inf), so its maxima need not quiet NaN inputs first (saves vector-ALU work per key block).
HIP_EXTRA = {"prefill.hip": ["-fno-honor-nans"]}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return r


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    """Compile every source and link librswa.so; returns its path. Always recompiles."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []
        extra += HIP_EXTRA.get(src, [])
        jobs.append(([HIPCC, *HIP_FLAGS, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj],
                     obj))
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        jobs.append((["g++", *COMMON, "-Wall", "-Wextra", "-c", os.path.join(CSRC, src), "-o", obj],
                     obj))
    with ThreadPoolExecutor(min(8, len(jobs))) as ex:
        results = list(ex.map(lambda j: _run(j[0], verbose), jobs))
    if resource_usage:
        for r in results:
            if r.stderr.strip():
                print(r.stderr, file=sys.stderr)
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, *HIP_FLAGS, "-shared", "-fPIC", "-o", tmp, *[o for _, o in jobs]], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, resource_usage="--usage" in sys.argv))
