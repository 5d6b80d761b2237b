"""The benchmark's JSON line on a GPU: bench.py run as the driver runs it
prints one line that keeps the benchmark contract."""
import pytest

pytestmark = pytest.mark.gpu


def test_bench_line_contract():
    """bench.py, run as the driver runs it (here with few launches and the
    optional tables off), prints one JSON line with every field of the
    benchmark contract: the metric and its value, the timing counts, the
    workload, the roofline object (bound, achieved, peak, unit, frac,
    traffic) for the dominant kernel and the CPU baseline (the oracle,
    with its core count and sample), and the metric's three parts."""
    import json
    import os
    import subprocess
    import sys
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--steps", "5", "--warmup", "5",
                          "--no-table", "--no-sweep", "--no-ladder", "--no-ceilings", "--cpu-seconds", "0.5",
                          "--part-cpu-seconds", "0.2"], capture_output=True, text=True, timeout=240)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [l for l in res.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, res.stdout[-2000:]
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline", "metric_parts"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 5 and d["higher_is_better"] is True
    assert d["config"]["workload"] == "fp16_4096" and d["dtype"] == "f16" and d["unit"] == "TFLOP/s"
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert abs(d["value"] - 2.0 * 4096 ** 3 / (d["ms_per_step"] * 1e-3) / 1e12) < 0.01 * d["value"]
    r = d["roofline"]
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert "traffic" in r
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["cores"] >= 1 and c["value"] > 0 and c["sample"]
    assert set(d["metric_parts"]) == {"fp16_4096", "int8_4096", "fp16_skinny"}
