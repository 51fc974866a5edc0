"""The host code behind the C ABI (argument validation, overlap arithmetic on
caller strides, the plan cache, the tile planner, the allocation-free plan
table) under AddressSanitizer and UndefinedBehaviorSanitizer: api.cpp and
planner.cpp are rebuilt by g++ with -fsanitize=address,undefined (the GPU
code is not sanitised), and the CPU tests that drive them -- test_abi.py and
test_planner.py -- run again in a subprocess against that library.  Any
sanitizer report fails the run."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="needs g++ and hipcc")


def test_abi_and_planner_under_asan_and_ubsan():
    from packed_varlen_attention_head_amd import build

    lib = build.build_sanitized()
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "host code is not instrumented"
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    env = dict(os.environ, LD_PRELOAD=asan, H3A_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_abi.py", "tests/test_planner.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    print(out[-3000:])
    assert "AddressSanitizer" not in out and "runtime error" not in out
    assert r.returncode == 0
