"""The library's host code under AddressSanitizer with UndefinedBehaviorSanitizer,
and under ThreadSanitizer.

The host API (csrc/tdg_api.hip: validation, planner, plan cache, split-K
planning, tile arithmetic; it holds no kernels) is compiled host-only with
the sanitizers and linked with the kernel objects of the last build into a
library copy in a temporary folder.  tests/c_abi/tdg_host_sanitize.cc then
drives every host path from eight threads; any sanitizer report fails it.
CPU only: no kernel is launched, and calls that pass validation are made only
where no device exists (they stop at the device check)."""
import glob
import os
import subprocess

import pytest

from conftest import no_device_only

import tiled_dense_gemm_loop_amd.build as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "c_abi", "tdg_host_sanitize.cc")
ROCM = "/opt/rocm"
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")
# (each -fsanitize= goes to the host compilation only)
SANITIZERS = {
    "address_undefined": (["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                           "-Xarch_host", "-fno-sanitize-recover=undefined"],
                          "libclang_rt.asan-x86_64.so",
                          {"ASAN_OPTIONS": "detect_leaks=0", "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}),
    "thread": (["-Xarch_host", "-fsanitize=thread"], "libclang_rt.tsan-x86_64.so",
               {"TSAN_OPTIONS": "halt_on_error=1:report_signal_unsafe=0"}),
}


def _run(cmd, env=None, timeout=300):
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout, env=env)
    assert res.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), res.stdout[-3000:], res.stderr[-6000:])
    return res.stdout


@no_device_only
@pytest.mark.parametrize("kind", sorted(SANITIZERS))
def test_host_code_under_sanitizers(tmp_path, kind):
    flags, runtime, env_extra = SANITIZERS[kind]
    others = [os.path.join(b.OBJ_DIR, obj) for src, _, obj in b.UNITS if src != "tdg_api.hip"]
    if not all(os.path.exists(o) for o in others):
        pytest.skip("build the library first (__graft_entry__.build())")
    api = str(tmp_path / "tdg_api_san.o")
    _run([b.HIPCC, "--offload-arch=gfx950", "--cuda-host-only", "-O1", "-g", "-std=c++17", "-fPIC",
          "-fno-omit-frame-pointer"] + flags +
         ["-I" + b.INCLUDE, "-I" + b.CSRC, "-c", os.path.join(b.CSRC, "tdg_api.hip"), "-o", api])
    lib = str(tmp_path / "libtdgemm.so")
    _run([b.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libsan"] + flags +
         ["-o", lib, api] + others)
    rt = os.path.dirname(subprocess.run([CLANG, "-print-file-name=" + runtime],
                                        capture_output=True, text=True).stdout.strip())
    exe = str(tmp_path / "tdg_host_sanitize")
    _run([CLANG, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-shared-libsan"] +
         [f for f in flags if f != "-Xarch_host"] + ["-D__HIP_PLATFORM_AMD__",
          "-I" + ROCM + "/include", "-I" + b.INCLUDE, DRIVER, "-L" + str(tmp_path), "-ltdgemm",
          "-L" + ROCM + "/lib", "-lamdhip64", "-lpthread",
          "-Wl,-rpath," + ":".join([str(tmp_path), ROCM + "/lib", rt]), "-o", exe])
    env = dict(os.environ, **env_extra)
    out = _run([exe], env=env)
    assert "sanitized host checks passed" in out, out
