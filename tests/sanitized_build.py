"""Host-sanitized build of the C ABI, for the CPU tests.

Compiles the library's sources with AddressSanitizer and UndefinedBehavior-
Sanitizer on the host side only (the device code is built as usual, without
them) and links them into one shared library with the clang sanitizer
runtime.  The CPU tests call only what runs on the host: argument checks,
workspace plans and the size queries.

Also builds a tiny planted-bug library (an out-of-bounds heap read) the same
way, so a test can confirm that the harness reports such errors.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "lm_head_top_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")

# host-side sanitizer flags; each -fsanitize= goes to the host pass only
HOST_SAN = [*"-Xarch_host -fsanitize=address".split(), *"-Xarch_host -fsanitize=undefined".split(),
            *"-Xarch_host -fno-sanitize-recover=all".split(), *"-Xarch_host -fno-omit-frame-pointer".split()]
CXX_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def asan_runtime():
    """Path of clang's shared ASan runtime (it carries the UBSan handlers too), or None."""
    c = sorted(glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux",
                                      "libclang_rt.asan-x86_64.so")))
    return c[-1] if c else None


def available() -> bool:
    return os.path.exists(HIPCC) and os.path.exists(CLANGXX) and asan_runtime() is not None


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{r.stdout}{r.stderr}")


def build(out_dir: str) -> str:
    """Builds libkdtopk_hostsan.so in out_dir; returns its path."""
    os.makedirs(out_dir, exist_ok=True)
    inc = [f"-I{INCLUDE}", f"-I{CSRC}"]
    jobs, objs = [], []
    for src in ("kd_kernels.hip", "kd_topk_select.hip", "kd_capi.hip"):
        o = os.path.join(out_dir, src + ".o")
        jobs.append([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                     "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                     "-Wno-unused-command-line-argument", *HOST_SAN, *inc, "-c",
                     os.path.join(CSRC, src), "-o", o])
        objs.append(o)
    o = os.path.join(out_dir, "kd_plan.cpp.o")
    jobs.append([CLANGXX, "-O1", "-g", "-std=c++17", "-fPIC", *CXX_SAN, *inc, "-c",
                 os.path.join(CSRC, "kd_plan.cpp"), "-o", o])
    objs.append(o)
    with concurrent.futures.ThreadPoolExecutor(len(jobs)) as ex:
        for f in [ex.submit(_run, j) for j in jobs]:
            f.result()
    lib = os.path.join(out_dir, "libkdtopk_hostsan.so")
    _run([HIPCC, "-shared", "-fPIC", *CXX_SAN, "-shared-libsan", *objs, "-o", lib])
    return lib


PLANTED = r"""
#include <stdlib.h>
extern "C" int kd_planted_oob_read(int n) {
  int* a = (int*)malloc(n * sizeof(int));
  for (int i = 0; i < n; ++i) a[i] = i;
  int s = a[n];  /* one past the end */
  free(a);
  return s;
}
"""


def build_planted(out_dir: str) -> str:
    os.makedirs(out_dir, exist_ok=True)
    src = os.path.join(out_dir, "planted.cpp")
    with open(src, "w") as f:
        f.write(PLANTED)
    lib = os.path.join(out_dir, "libplanted.so")
    _run([CLANGXX, "-O0", "-g", "-shared", "-fPIC", *CXX_SAN, "-shared-libsan", src, "-o", lib])
    return lib


def env() -> dict:
    """Environment for a child process that loads a sanitized library."""
    rt = asan_runtime()
    e = dict(os.environ)
    e["LD_PRELOAD"] = rt
    e["LD_LIBRARY_PATH"] = os.path.dirname(rt) + os.pathsep + e.get("LD_LIBRARY_PATH", "")
    # leaks: the HIP and Python runtimes keep allocations until exit by design
    e["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:abort_on_error=1"
    e["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return e
