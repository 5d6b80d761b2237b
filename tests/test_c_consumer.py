"""The C ABI from plain C: include/tdgemm.h compiles as C99 (pedantic) and as
C++11, and tests/c_abi/tdg_c_consumer.c, which reaches the library only
through that header and the HIP runtime's C API, builds with gcc, runs its
host checks without a GPU, and on a GPU runs INT8 / FP16 / FP32 products
against the CPU oracle (liboracle_gemm.so)."""
import os
import subprocess

import pytest

import tiled_dense_gemm_loop_amd as tdg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tdgemm.h")
SOURCE = os.path.join(ROOT, "tests", "c_abi", "tdg_c_consumer.c")
ROCM = "/opt/rocm"


def _run(cmd, timeout=120):
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout)
    assert res.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), res.stdout, res.stderr)
    return res.stdout


@pytest.fixture(scope="module")
def consumer(tmp_path_factory):
    import oracle
    oracle_lib = oracle._load()._name
    pkg_dir = os.path.dirname(tdg.LIB_PATH)
    oracle_dir = os.path.dirname(oracle_lib)
    assert os.path.exists(tdg.LIB_PATH), "build the library first (__graft_entry__.build())"
    out = str(tmp_path_factory.mktemp("c_abi") / "tdg_c_consumer")
    _run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
          "-I" + ROCM + "/include", "-I" + os.path.join(ROOT, "include"), SOURCE,
          "-L" + pkg_dir, "-ltdgemm", "-L" + oracle_dir, "-loracle_gemm",
          "-L" + ROCM + "/lib", "-lamdhip64", "-lm",
          "-Wl,-rpath," + ":".join([pkg_dir, oracle_dir, ROCM + "/lib"]), "-o", out])
    return out


def test_header_is_c99_and_cxx11():
    _run(["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-fsyntax-only",
          "-x", "c", HEADER])
    _run(["g++", "-std=c++11", "-pedantic", "-Wall", "-Wextra", "-Werror", "-fsyntax-only",
          "-x", "c++", HEADER])


def test_c_consumer_host_checks(consumer):
    out = _run([consumer, "host"])
    assert "host checks passed" in out


@pytest.mark.gpu
def test_c_consumer_gpu_products(consumer):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    out = _run([consumer, "gpu"])
    assert "gpu checks passed" in out and out.count(" ok\n") == 6
