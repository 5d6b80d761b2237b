"""The measurement harness's host logic (bench.py), without a GPU: the
roofline classification and throughput arithmetic of the benchmark's
workloads, the lookup of HBM traffic from the committed rocprofv3 summaries
(which must return nothing once the kernel source differs from the one the
counters were taken on), the bounded oracle sample of the CPU baseline, and
the refusal of more than one GPU."""
import os
import shutil
import subprocess
import sys

import pytest

import bench
import synthetic_inputs as si

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_roofline_classes_of_the_workloads():
    """"Analyze Kernel Bottleneck", Step 2: below the balance point is
    memory-bound.  The skinny product sits far below it; the 4096^3 products
    and FP32 far above."""
    for name, bound in (("fp16_4096", "mfma"), ("int8_4096", "mfma"), ("fp32_4096", "mfma"),
                        ("fp16_skinny", "hbm")):
        w = si.WORKLOADS[name]
        ops = 2.0 * w.M * w.N * w.K
        es = bench.ELEM_BYTES[w.dtype]
        alg = (w.M * w.K + w.K * w.N) * es + w.M * w.N * 4
        # operations and bytes per launch against GOP/s and GB/s
        assert bench.roofline_bound(ops, alg, bench.PEAK[w.dtype] * 1e3, bench.HBM_PEAK_GBS) == bound, name


def test_throughput_arithmetic():
    w = si.WORKLOADS["fp16_4096"]
    tflops, gbs = bench.throughput(w, 0.1)   # 100 us
    assert tflops == pytest.approx(2.0 * 4096 ** 3 / 1e-4 / 1e12)
    assert gbs == pytest.approx((2 * 4096 * 4096 * 2 + 4096 * 4096 * 4) / 1e-4 / 1e9)
    s = si.WORKLOADS["fp16_skinny"]
    _, gbs = bench.throughput(s, 0.04)
    assert gbs == pytest.approx(273678336 / 4e-5 / 1e9)


def test_profiled_traffic_follows_the_kernel_source(tmp_path, monkeypatch):
    """The committed FP16 4096^3 summary gives the headline's traffic for the
    current kernel source; a copy of the tree whose kernel source differs by
    one byte gets None, as does a configuration no summary covers and a
    workload whose summaries name the same configuration but another
    product (the ragged 4000^3 runs the same tile)."""
    desc = None
    for line in open(os.path.join(ROOT, "profiles", "gemm_fp16_4096_direct_lds_s2_w8_256x256x64.md")):
        if line.startswith("Config: "):
            desc = line[len("Config: "):].strip()
    assert desc
    t = bench.profiled_traffic("fp16_4096", desc)
    assert t is not None and t > 134217728          # at least the algorithmic bytes
    assert bench.profiled_traffic("fp16_4096", desc + " (not built)") is None
    ragged = bench.profiled_traffic("fp16_ragged", desc)
    assert ragged is None or ragged != t
    assert bench.profiled_traffic("int8_256", desc) is None
    fake = tmp_path / "tree"
    (fake / "tiled_dense_gemm_loop_amd" / "csrc").mkdir(parents=True)
    shutil.copytree(os.path.join(ROOT, "profiles"), fake / "profiles")
    src = open(os.path.join(ROOT, "tiled_dense_gemm_loop_amd", "csrc", "tdg_kernels.hpp"), "rb").read()
    (fake / "tiled_dense_gemm_loop_amd" / "csrc" / "tdg_kernels.hpp").write_bytes(src + b"\n")
    monkeypatch.setattr(bench, "ROOT", str(fake))
    assert bench.profiled_traffic("fp16_4096", desc) is None


def test_oracle_sample_is_bounded_and_whole_rows():
    """The CPU baseline times the oracle on the first rows of C: all of them
    when that is quick, else a multiple of the thread count, and reports
    operations per second over the rows it ran."""
    import oracle
    w = si.WORKLOADS["int8_256"]
    A, B = w.operands()
    ops, rows, secs = bench.oracle_rate(w, A, B, 0.5, oracle.host_threads())
    assert rows == w.M and secs > 0 and ops == pytest.approx(2.0 * rows * w.N * w.K / secs)
    w = si.WORKLOADS["fp16_1024"]
    A, B = w.operands()
    threads = oracle.host_threads()
    ops, rows, secs = bench.oracle_rate(w, A, B, 0.05, threads)
    assert 1 <= rows <= w.M and (rows == w.M or rows % threads == 0 or rows == min(threads, w.M))
    assert ops > 0


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode != 0
    assert "one GPU" in (res.stdout + res.stderr)
