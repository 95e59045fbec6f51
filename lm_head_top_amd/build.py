"""Builds libkdtopk.so (the HIP library behind include/kdtopk.h) for gfx950, in-tree.

Usage: python -m lm_head_top_amd.build [-v]
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libkdtopk.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
# the same library with device-side bounds checks on the cache-entry
# scatters and gathers (KD_DEBUG_BOUNDS), for debugging only
DEBUG_LIB_NAME = "libkdtopk_debug.so"
DEBUG_LIB_PATH = os.path.join(HERE, DEBUG_LIB_NAME)
ARCH = "gfx950"

HIP_SOURCES = ["kd_kernels.hip", "kd_topk_select.hip", "kd_capi.hip"]
HOST_SOURCES = ["kd_plan.cpp"]

# Packed-FP32 VALU ops are disabled for all device code.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else (shutil.which("hipcc") or "hipcc")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    """Compiles every source and links the shared library and its debug
    variant; returns the library's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    hipcc = _hipcc()
    inc = [f"-I{INCLUDE}", f"-I{CSRC}"]
    jobs = []
    objs = {LIB_PATH: [], DEBUG_LIB_PATH: []}
    for lib, defs, tag in ((LIB_PATH, [], ""), (DEBUG_LIB_PATH, ["-DKD_DEBUG_BOUNDS=1"], ".debug")):
        for src in HIP_SOURCES:
            obj = os.path.join(BUILD_DIR, src + tag + ".o")
            objs[lib].append(obj)
            jobs.append([hipcc, "-x", "hip", *HIP_FLAGS, *defs, *inc, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        for lib in objs:
            objs[lib].append(obj)
        jobs.append(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", *inc, "-c",
                     os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as ex:
        for f in [ex.submit(_run, j, verbose) for j in jobs]:
            f.result()
    for lib, lobjs in objs.items():
        tmp = lib + ".tmp"
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *lobjs, "-o", tmp], verbose)
        os.replace(tmp, lib)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
