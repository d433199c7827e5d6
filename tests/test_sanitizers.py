"""The host-side C and C++ code under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

* The fp64 oracle (oracle/attn_oracle.c, oracle/attn_bwd_oracle.c), driven
  by tests/sanitize_oracle.c through every index path on small inputs:
  ragged shapes, both masks, row, head, query and key selections, and the
  argument checks, each value checked against exact properties.
* The index arithmetic of the prefill kernel's layout (tests/layout_check.cpp
  over io_aware_amd/csrc/fa_layout.h).

Both are built with gcc / g++ with -fsanitize=address,undefined and
-fno-sanitize-recover=all, so any finding fails the run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="3")

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                                reason="gcc / g++ not installed")


def run(exe):
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=ENV, timeout=300)
    assert res.returncode == 0 and res.stdout.strip().endswith("OK"), res.stdout[-3000:] + res.stderr[-3000:]


def test_oracle_under_sanitizers(tmp_path):
    exe = tmp_path / "sanitize_oracle"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-fopenmp"] + SAN +
                   [os.path.join(ROOT, "tests", "sanitize_oracle.c"), os.path.join(ROOT, "oracle", "attn_oracle.c"),
                    os.path.join(ROOT, "oracle", "attn_bwd_oracle.c"), "-o", str(exe), "-lm"], check=True)
    run(exe)


def test_layout_check_under_sanitizers(tmp_path):
    exe = tmp_path / "layout_check"
    subprocess.run(["g++", "-std=c++17", "-Wall"] + SAN +
                   ["-I", os.path.join(ROOT, "io_aware_amd", "csrc"), os.path.join(ROOT, "tests", "layout_check.cpp"),
                    "-o", str(exe)], check=True)
    run(exe)
