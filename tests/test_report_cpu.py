"""The bottleneck report generator runs on a benchmark detail file and the
committed rocprofv3 summaries, and writes every section of the report
layout of "Analyze Kernel Bottleneck", Step 8."""
import json
import os

from tiled_dense_gemm_loop_amd import report

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _detail():
    """A detail file in the shape bench.py writes (figures of one run)."""
    parts = {"fp16_4096": {"value": 1150.0, "unit": "TFLOP/s", "us": 119.5, "peak": 2500.0, "frac": 0.46},
             "int8_4096": {"value": 2100.0, "unit": "TOP/s", "us": 65.4, "peak": 5000.0, "frac": 0.42},
             "fp16_skinny": {"value": 6400.0, "unit": "GB/s", "us": 42.8, "peak": 8000.0, "frac": 0.8}}
    line = {"steps": 20, "warmup": 5, "metric_parts": parts}

    def kern(bm, bn, bk, waves, stages, ratio, need, mpl, lds, grid, vgprs, wg):
        return {"config": {"bm": bm, "bn": bn, "bk": bk, "waves": waves, "lds_stages": stages, "variant": 3},
                "plan": {"ratio": ratio, "band": 2, "lds_bytes": lds, "wg_per_cu": wg, "num_tiles": 64,
                         "grid": grid, "need_bytes_per_clk": need, "mfma_per_load": mpl, "pipelined": 1},
                "resources": {"vgprs": vgprs, "spill_bytes": 0, "lds_bytes": lds, "threads": waves * 64,
                              "wg_per_cu": wg}}
    return {"line": line, "measured_ceilings": {"mfma_f16_tflops": 1700.0, "mfma_i8_tops": 3300.0,
                                                "copy_gbs": 5600.0},
            "kernels": {"fp16_4096": kern(256, 256, 64, 8, 2, 128.0, 32.0, 4.0, 131072, 256, 239, 1),
                        "int8_4096": kern(256, 256, 128, 8, 2, 256.0, 32.0, 4.0, 131072, 256, 247, 1),
                        "fp16_skinny": kern(64, 64, 64, 4, 4, 32.0, 128.0, 1.0, 65536, 256, 48, 2),
                        "int8_256": kern(64, 64, 128, 4, 4, 64.0, 128.0, 1.0, 65536, 16, 68, 2),
                        "fp16_1024": kern(64, 64, 64, 4, 4, 32.0, 128.0, 1.0, 65536, 256, 68, 2),
                        "fp32_4096": kern(256, 256, 32, 8, 2, 64.0, 4.0, 4.0, 131072, 256, 200, 1)},
            # the small configurations are timed per call and from HIP graphs
            "variants": {"int8_256": {"pipelined": {"us": 5.3}, "graph": {"pipelined": {"us": 3.1}}},
                         "fp16_1024": {"pipelined": {"us": 7.0}, "graph": {"pipelined": {"us": 6.8}}},
                         "fp32_4096": {"pipelined": {"us": 921.0}}}}


def test_report_has_every_section(tmp_path):
    profiles = os.path.join(ROOT, "profiles")
    det = tmp_path / "detail.json"
    det.write_text(json.dumps(_detail()))
    out = tmp_path / "out"
    out.mkdir()
    for f in os.listdir(profiles):
        if f.startswith("gemm_"):
            (out / f).write_text(open(os.path.join(profiles, f)).read())
    assert report.main([str(det), str(out)]) == 0
    for wl in ("fp16_4096", "int8_4096", "fp16_skinny", "int8_256", "fp16_1024", "fp32_4096"):
        text = (out / ("report_%s.md" % wl)).read_text()
        for section in ("## Baseline", "## Roofline classification", "## Occupancy", "## Compute / load ratio",
                        "## Instruction mix", "## LDS cliff", "## Recommended optimizations"):
            assert section in text, (wl, section)
        bound = {"fp16_skinny": "memory-bound", "int8_256": "latency-bound",
                 "fp16_1024": "latency-bound"}.get(wl, "compute-bound")
        assert "**%s**" % bound in text, (wl, bound)
        assert "1. " in text.split("## Recommended optimizations")[1]


def test_planner_command_line(capsys):
    """python -m tiled_dense_gemm_loop_amd.plan prints the planner's choice
    and its arithmetic for a product, and the form a call on given operands
    runs; no GPU is needed."""
    from tiled_dense_gemm_loop_amd import plan
    assert plan.main(["f16", "4096", "4096", "4096"]) == 0
    out = capsys.readouterr().out
    assert "256x256x64 tile, 8 waves, 2 LDS buffer(s), direct_lds" in out
    assert "ratio: 128.0 operations per byte" in out and "32.0 B per clock" in out
    assert "K loop: 64 tile(s), pipelined" in out and "split K: not predicted faster" in out
    assert plan.main(["i8", "256", "256", "65536"]) == 0
    assert "split K: 32 parts" in capsys.readouterr().out
    assert plan.main(["f16", "4095", "4095", "4095", "--misalign", "2"]) == 0
    assert "bounds-checked" in capsys.readouterr().out
    assert plan.main(["f32", "1", "1", "1"]) == 0
    assert "not pipelined (one K tile)" in capsys.readouterr().out
