"""Host check of the prefill kernel's LDS and MFMA-operand index arithmetic.

Builds tests/layout_check.cpp against io_aware_amd/csrc/fa_layout.h with g++
and runs it: every staging write in range and exactly once, every operand
read fetching the element the MFMA lane contract needs, and the workgroup
order a bijection.
"""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_layout_arithmetic(tmp_path):
    exe = tmp_path / "layout_check"
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror",
                    "-I", os.path.join(ROOT, "io_aware_amd", "csrc"),
                    os.path.join(ROOT, "tests", "layout_check.cpp"), "-o", str(exe)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True)
    assert res.returncode == 0 and res.stdout.strip().endswith("OK"), res.stdout + res.stderr
