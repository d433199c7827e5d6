"""Build ``libfa.so`` (the C-ABI library of HIP kernels) for gfx950.

Every source under ``csrc/`` is compiled by hipcc for gfx950 only, with
packed-fp32 instruction selection disabled, into ``_build/`` and linked in
place as ``io_aware_amd/libfa.so``.  ``build()`` always recompiles.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa.so")
SOURCES = ["fa_api.hip", "fa_prefill.hip", "fa_f32.hip", "fa_decode.hip", "fa_backward.hip", "fa_fp8.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm under /opt/rocm)")


COMPILE_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-c", os.path.join(CSRC, src), "-o", obj] + COMPILE_FLAGS
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("compiling %s failed:\n%s\n%s" % (src, " ".join(cmd), res.stderr))
    return obj


def build(jobs: int = 4) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "--offload-arch=gfx950", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("linking libfa.so failed:\n%s\n%s" % (" ".join(cmd), res.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
