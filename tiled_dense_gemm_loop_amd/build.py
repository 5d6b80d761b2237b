"""Build libtdgemm.so, the gfx950 GEMM library, in-tree with hipcc.

The kernel tables for the three dtypes are separate translation units and are
compiled in parallel with the host API and the copy/transpose ladder.  All
HIP code is compiled for gfx950 only, with packed-FP32 instruction selection
turned off.
"""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libtdgemm.so")
OBJ_DIR = os.path.join(PKG, "_build")  # object files of the last build
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE, "-I" + CSRC,
]

UNITS = [
    ("tdg_kernels.hip", ["-DTDG_BUILD_DT=0"], "tdg_kernels_f16.o"),
    ("tdg_kernels.hip", ["-DTDG_BUILD_DT=1"], "tdg_kernels_i8.o"),
    ("tdg_kernels.hip", ["-DTDG_BUILD_DT=2"], "tdg_kernels_f32.o"),
    ("tdg_api.hip", [], "tdg_api.o"),
    ("tdg_move.hip", [], "tdg_move.o"),
    ("tdg_probe.hip", [], "tdg_probe.o"),
    ("tdg_reduce.hip", [], "tdg_reduce.o"),
    ("tdg_noalloc.hip", [], "tdg_noalloc.o"),
]


def _compile(unit, outdir):
    src, extra, obj = unit
    out = os.path.join(outdir, obj)
    cmd = [HIPCC] + COMMON + extra + ["-c", os.path.join(CSRC, src), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), res.stderr))
    return out


def build_library(verbose: bool = False) -> str:
    """Compile every HIP source and link libtdgemm.so next to this file.  The
    objects stay in OBJ_DIR, where the host-code sanitizer test links them
    with an instrumented copy of the host API."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(UNITS)) as pool:
        objs = list(pool.map(lambda u: _compile(u, OBJ_DIR), UNITS))
    tmp_lib = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp_lib] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), res.stderr))
    os.replace(tmp_lib, LIB_PATH)
    if verbose:
        print("built", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build_library(verbose=True)
