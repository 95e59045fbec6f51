"""The C ABI from plain C: include/kdtopk.h compiles as C99 with warnings as
errors, and a C program linked against libkdtopk.so sizes a workspace, checks
arguments and names statuses through it (host-only calls, no device needed).
The numbers it prints must match the same calls made through ctypes."""
import os
import shutil
import subprocess

import pytest

import lm_head_top_amd as kd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

C_SRC = r"""
#include <stdio.h>
#include "kdtopk.h"

int main(void) {
  /* the toy LM head and the very-long workload */
  size_t a = kd_topk_kl_workspace_size(8192, 4096, 131072, 100, 1024);
  size_t b = kd_topk_kl_workspace_size(262144, 4096, 131072, 100, 4096);
  /* a rejected call returns its status before any HIP call */
  kd_status s = kd_topk_kl_forward(NULL, NULL, NULL, NULL, 1, 8, 8, 1, 1.0f, 1, NULL, NULL, NULL,
                                   NULL, 0, NULL);
  printf("%zu %zu %d %s\n", a, b, (int)s, kd_status_string(s));
  return s == KD_ERR_INVALID_ARG ? 0 : 1;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc missing")
def test_header_is_c99_and_links(tmp_path):
    if not os.path.exists(kd.lib_path()):
        pytest.skip("libkdtopk.so not built")
    src = tmp_path / "client.c"
    src.write_text(C_SRC)
    exe = tmp_path / "client"
    libdir = os.path.dirname(kd.lib_path())
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", f"-I{ROOT}/include", str(src),
           f"-L{libdir}", "-lkdtopk", f"-Wl,-rpath,{libdir}", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    a, b, s, *name = r.stdout.split()
    assert int(a) == kd.workspace_size(8192, 4096, 131072, 100, 1024)
    assert int(b) == kd.workspace_size(262144, 4096, 131072, 100, 4096)
    assert int(s) == 1 and " ".join(name) == "invalid argument"
