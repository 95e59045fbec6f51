"""The host side of the C ABI under AddressSanitizer and UndefinedBehavior-
Sanitizer (CPU only, no device code): every host test of the ABI and of the
binding's checks runs again against a sanitized build, in a child process
that preloads the sanitizer runtime.  A planted out-of-bounds read in a tiny
library built the same way must be reported, so a clean run means something."""
import ctypes
import os
import subprocess
import sys

import pytest

from tests import sanitized_build as SB

pytestmark = pytest.mark.skipif(not SB.available(), reason="hipcc, clang++ or the ASan runtime is missing")


@pytest.fixture(scope="module")
def san_dir(tmp_path_factory):
    return str(tmp_path_factory.mktemp("hostsan"))


def test_harness_reports_a_planted_out_of_bounds_read(san_dir):
    lib = SB.build_planted(san_dir)
    code = f"import ctypes; ctypes.CDLL({lib!r}).kd_planted_oob_read(4)"
    r = subprocess.run([sys.executable, "-c", code], env=SB.env(), capture_output=True, text=True,
                       timeout=300)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr


def test_host_abi_suites_are_clean_under_asan_and_ubsan(san_dir):
    lib = SB.build(san_dir)
    tests = [os.path.join(SB.HERE, f) for f in ("test_abi_host.py", "test_binding_checks.py")]
    r = subprocess.run([sys.executable, os.path.join(SB.HERE, "sanitized_runner.py"), lib, "-q", "-m",
                        "not gpu", "-p", "no:cacheprovider", *tests],
                       env=SB.env(), capture_output=True, text=True, timeout=900, cwd=SB.ROOT)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout
