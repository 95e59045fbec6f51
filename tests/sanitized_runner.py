"""Runs pytest with the binding pointed at a host-sanitized build of the
library (the path in the first argument).  Started by test_abi_sanitized.py
in a child process whose environment preloads the sanitizer runtime."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import lm_head_top_amd as kd  # noqa: E402

LIB = sys.argv[1]
kd.lib_path = lambda: LIB

import pytest  # noqa: E402

sys.exit(pytest.main(sys.argv[2:]))
