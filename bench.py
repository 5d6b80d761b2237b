"""Benchmark of the software-pipelined tiled GEMM on one MI355X.

One step = one C = A . B call on the headline workload (FP16 inputs, FP32
accumulate, M = N = K = 4096) with the operands already resident in HBM.
Timing uses HIP events recorded on the stream the kernels are launched on
(torch's current stream), bracketing exactly --steps launches after
--warmup untimed ones ("Analyze Kernel Bottleneck", Step 1: event timing
after warm-up, effective GFLOPS = 2*M*N*K / t).  After the warm-ups and a
synchronize, a ~150 us spin kernel is enqueued before the start event, so
the timed launches are queued back to back when timing begins.

Printed on stdout: ONE short JSON line with the headline value, the roofline
object of its kernel (with the metric's three parts -- FP16 and INT8 4096^3
against the dense MFMA peak, the skinny FP16 product against HBM -- under
roofline.parts and metric_parts), and the CPU oracle timed on bounded samples
on this host's cores, per configuration.  The side-by-side table of every
workload x loop variant (single-buffer, register prefetch, direct-to-LDS),
the tile sweep, the cold-cache runs, the copy / transpose ladder and the
measured ceilings go to stderr, and with --detail-out to a JSON file.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synthetic_inputs as si  # noqa: E402

METRIC = "GEMM TFLOPS/TOPS at 4096³ (FP16, INT8) + % of MFMA peak; skinny GB/s % HBM"
PEAK = {"f16": 2500.0, "i8": 5000.0, "f32": 157.3}   # dense MFMA, TFLOP/s and TOP/s
HBM_PEAK_GBS = 8000.0


def balance_point(peak_gops: float, bw_gbs: float) -> float:
    """Machine balance in operations per byte: peak compute / peak bandwidth
    ("Analyze Kernel Bottleneck", Step 2)."""
    return peak_gops / bw_gbs


def roofline_bound(ops: float, alg_bytes: float, peak_gops: float, bw_gbs: float) -> str:
    """'hbm' when the arithmetic intensity (operations per unique byte of HBM
    traffic) is below the machine balance, else 'mfma'."""
    return "hbm" if ops / alg_bytes < balance_point(peak_gops, bw_gbs) else "mfma"


def profiled_traffic(workload: str, kernel_desc: str):
    """HBM bytes per launch from the committed rocprofv3 summary of this
    workload in profiles/ (gemm_<workload>_*.md; calibrated FETCH_SIZE +
    WRITE_SIZE), or None when no summary of it matches this kernel
    configuration and the current kernel source."""
    import glob
    import hashlib
    src = os.path.join(ROOT, "tiled_dense_gemm_loop_amd", "csrc", "tdg_kernels.hpp")
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "gemm_%s_*.md" % workload))):
        fields = {}
        for line in open(path):
            for key in ("Kernel source sha256[:16]: ", "Config: "):
                if line.startswith(key):
                    fields[key] = line[len(key):].strip()
            if "traffic_bytes: " in line:
                fields["traffic"] = float(line.split("traffic_bytes: ")[1].split()[0])
        if fields.get("Kernel source sha256[:16]: ") == digest and \
                fields.get("Config: ") == kernel_desc and "traffic" in fields:
            return fields["traffic"]
    return None


def parse():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    # A launch is ~0.1 ms.  The clocks ramp up over the first tens of
    # milliseconds under load (FP16 4096^3 on one box: 126 us per launch over
    # the first 50 launches after 50 warm-ups, a steady 110.8 us after about
    # 350), so 400 untimed launches come first and the next 400 (~45 ms) are
    # timed at the steady state.
    p.add_argument("--steps", type=int, default=400)
    p.add_argument("--warmup", type=int, default=400)
    p.add_argument("--workload", default="fp16_4096", choices=sorted(si.WORKLOADS))
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-table", action="store_true", help="skip the per-workload variant table")
    p.add_argument("--no-parts", action="store_true",
                   help="skip timing the metric's other parts (INT8 4096^3, skinny)")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--no-ladder", action="store_true", help="skip the copy/transpose ladder")
    p.add_argument("--no-ceilings", action="store_true",
                   help="skip the measured MFMA ceilings (MFMA-only probe)")
    p.add_argument("--no-sweep", action="store_true",
                   help="skip the FP16 4096^3 sweep over every built configuration")
    p.add_argument("--sweep-steps", type=int, default=50,
                   help="timed launches per configuration in the sweep")
    p.add_argument("--copy-calib-mib", type=int, default=0,
                   help="also run one device copy of this many MiB (counter calibration)")
    p.add_argument("--part-cpu-seconds", type=float, default=2.0,
                   help="target CPU time of the oracle sample for each other configuration")
    p.add_argument("--detail-out", default=None,
                   help="also write the full record (variant table, sweep, ladder, ceilings, "
                        "cold runs) as JSON to this file; it always goes to stderr")
    return p.parse_args()


def device_operands(wl):
    import torch
    A, B = wl.operands()
    if wl.dtype == "f32":
        dA = torch.from_numpy(A).cuda()
        dB = torch.from_numpy(B).cuda()
        C = torch.empty((wl.M, wl.N), dtype=torch.float32, device="cuda")
    elif wl.dtype == "f16":
        dA = torch.from_numpy(A.view(np.int16)).cuda().view(torch.float16)
        dB = torch.from_numpy(B.view(np.int16)).cuda().view(torch.float16)
        C = torch.empty((wl.M, wl.N), dtype=torch.float32, device="cuda")
    else:
        dA = torch.from_numpy(A).cuda()
        dB = torch.from_numpy(B).cuda()
        C = torch.empty((wl.M, wl.N), dtype=torch.int32, device="cuda")
    return A, B, dA, dB, C


def launcher(tdg, wl, dA, dB, C, variant: str):
    fns = {"f16": (tdg.gemm_f16f32, tdg.gemm_f16f32_pipelined, tdg.gemm_f16f32_ex),
           "i8": (tdg.gemm_i8i32, tdg.gemm_i8i32_pipelined, tdg.gemm_i8i32_ex),
           "f32": (tdg.gemm_f32f32, tdg.gemm_f32f32_pipelined, tdg.gemm_f32f32_ex)}[wl.dtype]
    if variant == "pipelined":
        fn = fns[1]
        return lambda: fn(dA, dB, C)
    if variant == "single":
        fn = fns[0]
        return lambda: fn(dA, dB, C)
    cfg = {"reg_s1": dict(variant=tdg.TDG_VARIANT_REG_PREFETCH, lds_stages=1),
           "reg_s2": dict(variant=tdg.TDG_VARIANT_REG_PREFETCH, lds_stages=2),
           "direct": dict(variant=tdg.TDG_VARIANT_DIRECT_LDS, lds_stages=2)}[variant]
    fn = fns[2]
    return lambda: fn(dA, dB, C, cfg=cfg)


def hold_stream(us: float = 150.0) -> None:
    """Enqueue a short spin kernel on the current stream, so that the launches
    enqueued after it are already queued when the GPU reaches the next event:
    the timed region then holds only back-to-back kernels, not the host's
    latency for the first launch after a synchronize (which would be amortised
    over few launches: ~1.5-3% at 20 of them)."""
    import torch
    sleep = getattr(torch.cuda, "_sleep", None)
    if sleep is not None:
        sleep(int(us * 2400))  # cycles of a clock of about 2.4 GHz or less


def time_launches(run, steps: int, warmup: int) -> float:
    """Mean milliseconds per launch over `steps` back-to-back launches,
    bracketed by events on the launching (current) stream."""
    import torch
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    hold_stream()
    start.record()
    for _ in range(steps):
        run()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def graph_launches(run, per_graph: int = 20, replays: int = 20) -> float:
    """Mean milliseconds per launch when `per_graph` launches are captured in
    one HIP graph and the graph is replayed: the launch-bound small shapes
    then pay the graph's replay cost instead of one host call per launch."""
    import torch
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()  # warm the library's caches outside the capture
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            run()
    g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(replays):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / (replays * per_graph)


def individual_launches(run, count: int = 50) -> dict:
    """Median / min / max microseconds of `count` launches, each bracketed by
    its own pair of events on the launching stream."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(count)]
    for a, b in evs:
        a.record()
        run()
        b.record()
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    return {"count": count, "median_us": round(us[count // 2], 2), "min_us": round(us[0], 2),
            "max_us": round(us[-1], 2)}


ELEM_BYTES = {"f16": 2, "i8": 1, "f32": 4}
UNITS = {"f16": "TFLOP/s", "i8": "TOP/s", "f32": "TFLOP/s"}
DTYPE_CODE = {"f16": 0, "i8": 1, "f32": 2}


def cold_launches(tdg, wl, count: int = 20, scrub_mib: int = 512) -> dict:
    """Launches that start with cold caches.  Before each one a 512 MiB
    buffer (more than the 256 MB last-level cache holds) is either read
    (the caches then hold clean scrub data) or written (they then hold dirty
    lines, whose write-back the launch also pays for).  Only the launch
    itself is bracketed by events."""
    import torch
    A, B, dA, dB, C = device_operands(wl)
    run = launcher(tdg, wl, dA, dB, C, "pipelined")
    scrub = torch.ones(scrub_mib * (1 << 20) // 4, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")  # the 0-d sum of the scrub
    run()
    out = {"workload": wl.name, "scrub_mib": scrub_mib, "count": count}
    for mode in ("read", "write"):
        evs = []
        for i in range(count):
            if mode == "read":
                torch.sum(scrub, dim=0, out=sink)
            else:
                scrub.fill_(float(i))
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            run()
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        us = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
        med = us[count // 2]
        tops, gbs = throughput(wl, med * 1e-3)
        out["after_%s_scrub" % mode] = {"median_us": round(med, 2), "min_us": round(us[0], 2),
                                        "gbs": round(gbs, 1), "tops": round(tops, 1)}
    del A, B, dA, dB, C, scrub
    torch.cuda.empty_cache()
    return out


def throughput(wl, ms: float):
    ops = 2.0 * wl.M * wl.N * wl.K
    es = ELEM_BYTES[wl.dtype]
    alg_bytes = (wl.M * wl.K + wl.K * wl.N) * es + wl.M * wl.N * 4
    return ops / (ms * 1e-3) / 1e12, alg_bytes / (ms * 1e-3) / 1e9


def transpose_ladder(tdg):
    """The copy / transpose ladder ("fixing GPU kernels by hand"): effective
    bandwidth = 2 * n^2 * 4 bytes over the mean launch time, for the page's
    4096^2 float matrix (input and output fit the 256 MB last-level cache)
    and for 16384^2 (1 GiB each way, HBM-bound)."""
    import torch
    out = {}
    for n, steps in ((4096, 200), (16384, 40)):
        x = torch.randn(n, n, device="cuda")
        y = torch.empty(n, n, device="cuda")
        moved = 2.0 * n * n * 4
        rows = {"copy": time_launches(lambda: tdg.tdg_copy_f32(x, y), steps, 20)}
        for code, name in tdg.TRANSPOSE_NAMES.items():
            rows[name] = time_launches(lambda: tdg.tdg_transpose_f32(x, y, method=code), steps, 20)
        copy_ms = rows["copy"]
        out["%dx%d" % (n, n)] = {
            name: {"us": round(ms * 1e3, 2), "gbs": round(moved / (ms * 1e-3) / 1e9, 1),
                   "of_copy": round(copy_ms / ms, 3),
                   "of_hbm_peak": round(moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 3)}
            for name, ms in rows.items()}
        print("# ladder %dx%d %s" % (n, n, json.dumps(out["%dx%d" % (n, n)])), file=sys.stderr,
              flush=True)
        del x, y
        torch.cuda.empty_cache()
    return out


def measured_ceilings(tdg, ladder):
    """Second denominators: the MFMA rate the chip sustains with no memory
    traffic (tdg_mfma_probe, ~20 ms per launch, 5 launches after 2, so the
    power controller settles), the LDS read rate per CU of the fragment
    reads' instruction forms (tdg_lds_probe), and the bandwidth of the
    library's copy on a matrix far larger than the last-level cache."""
    import torch
    out = {}
    sink = torch.empty(tdg.tdg_mfma_probe_sink_floats(), dtype=torch.float32, device="cuda")
    for code, key, iters in ((tdg.TDG_DTYPE_F16F32, "mfma_f16_tflops", 80000),
                             (tdg.TDG_DTYPE_I8I32, "mfma_i8_tops", 80000),
                             (tdg.TDG_DTYPE_F32F32, "mfma_f32_tflops", 40000)):
        ms = time_launches(lambda: tdg.tdg_mfma_probe(code, iters, sink), 5, 2)
        out[key] = round(tdg.tdg_mfma_probe_ops(code, iters) / (ms * 1e-3) / 1e12, 1)
    for name, mode in tdg.LDS_PROBE_MODES.items():
        out["lds_%s_bytes_per_clk" % name] = round(tdg.tdg_lds_probe(mode, 4096), 1)
    if ladder and "16384x16384" in ladder:
        out["copy_gbs"] = ladder["16384x16384"]["copy"]["gbs"]
    print("# measured ceilings %s" % json.dumps(out), file=sys.stderr, flush=True)
    return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def tile_sweep(tdg, steps: int, warmup: int):
    """FP16 4096^3 on every built configuration (tile, waves, LDS ring, loop
    form): the planner's LDS budget, ratio and occupancy arithmetic
    ("Pipeline GPU Kernel", Step 1 and Step 2; "Analyze Kernel Bottleneck",
    Step 3 and Step 6) beside the runtime's view of the same kernel
    (registers, spills, LDS, resident workgroups per CU), with the rate each
    one reaches and its fraction of the dense MFMA peak."""
    import torch
    wl = si.WORKLOADS["fp16_4096"]
    _, _, dA, dB, C = device_operands(wl)
    code = DTYPE_CODE["f16"]
    rows = []
    for i in range(tdg.tdg_config_count(code)):
        cfg = tdg.tdg_config_at(code, i)
        res = tdg.tdg_config_resources(code, i)
        fig = tdg.tdg_tile_figures(code, cfg["bm"], cfg["bn"], cfg["bk"], cfg["waves"],
                                   cfg["lds_stages"], cfg["variant"], wl.M, wl.N, wl.K)
        ms = time_launches(lambda: tdg.gemm_f16f32_ex(dA, dB, C, cfg=cfg), steps, warmup)
        tf = 2.0 * wl.M * wl.N * wl.K / (ms * 1e-3) / 1e12
        rows.append({
            "tile": "%dx%dx%d" % (cfg["bm"], cfg["bn"], cfg["bk"]), "waves": cfg["waves"],
            "lds_stages": cfg["lds_stages"], "variant": tdg.VARIANT_NAMES[cfg["variant"]],
            "ratio": round(fig["ratio"], 1), "need_bytes_per_clk": round(fig["need_bytes_per_clk"], 1),
            "lds_kib": round(fig["lds_bytes"] / 1024.0, 1), "grid": fig["grid"],
            "wg_per_cu_planned": fig["wg_per_cu"], "wg_per_cu_runtime": res["wg_per_cu"],
            "vgprs": res["vgprs"], "spill_bytes": res["spill_bytes"],
            "us": round(ms * 1e3, 2), "tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK["f16"], 4)})
    del dA, dB, C
    torch.cuda.empty_cache()
    rows.sort(key=lambda r: -r["tflops"])
    return rows


def oracle_rate(wl, A, B, target_s: float, threads: int):
    """The oracle as it stands on a bounded sample of one workload: the first
    R rows of C, R chosen so that the run takes about target_s seconds on
    this host (all of C when that is quicker).  Returns (ops per second, rows,
    seconds)."""
    import oracle
    fn = {"f16": oracle.gemm_f16, "i8": oracle.gemm_i8, "f32": oracle.gemm_f32}[wl.dtype]
    probe_rows = min(wl.M, max(threads, 16))
    t0 = time.perf_counter()
    fn(A[:probe_rows], B, threads=threads)
    t_probe = time.perf_counter() - t0
    rows = int(min(wl.M, max(probe_rows, probe_rows * target_s / max(t_probe, 1e-6))))
    if rows < wl.M:
        rows = max(min(threads, wl.M), (rows // threads) * threads)
    t0 = time.perf_counter()
    fn(A[:rows], B, threads=threads)
    secs = time.perf_counter() - t0
    if rows < wl.M and secs < target_s / 3:  # the small probe overestimated the cost per row
        rows = int(min(wl.M, rows * target_s / max(secs, 1e-6)))
        if rows < wl.M:
            rows = max(threads, (rows // threads) * threads)
        t0 = time.perf_counter()
        fn(A[:rows], B, threads=threads)
        secs = time.perf_counter() - t0
    return 2.0 * rows * wl.N * wl.K / secs, rows, secs


def cpu_baseline(wl, A, B, target_s: float, part_s: float, part_names):
    """The oracle timed on this host's cores: the headline workload on a
    sample of about target_s seconds, every other named workload on one of
    about part_s seconds, and the FP16 1024^3 workload on one thread (a
    per-core figure)."""
    import oracle
    threads = oracle.host_threads()
    ops, rows, secs = oracle_rate(wl, A, B, target_s, threads)
    unit = UNITS[wl.dtype]
    per = {}
    for name in part_names:
        w = si.WORKLOADS[name]
        if name == wl.name:
            r_ops, r_rows, r_secs = ops, rows, secs
        else:
            a, b = w.operands()
            r_ops, r_rows, r_secs = oracle_rate(w, a, b, part_s, threads)
        per[name] = {"value": round(r_ops / 1e9, 3), "unit": "GOP/s", "cores": threads,
                     "sample": "rows 0..%d of C (%d x %d x %d, %.2f s)" % (
                         r_rows - 1, r_rows, w.N, w.K, r_secs)}
    small = si.WORKLOADS["fp16_1024"]
    sa, sb = small.operands()
    t0 = time.perf_counter()
    oracle.gemm_f16(sa, sb, threads=1)
    one = time.perf_counter() - t0
    return {"value": ops / 1e12, "unit": unit, "cores": threads, "kind": "oracle",
            "sample": "rows 0..%d of C (%d x %d x %d, %.1f s)" % (rows - 1, rows, wl.N, wl.K, secs),
            "cpu_model": cpu_model(),
            "one_thread_fp16_1024": {"seconds": round(one, 3),
                                     "tflops": round(2.0 * 1024 ** 3 / one / 1e12, 5)},
            "per_config": per}


def kernel_record(tdg, wl) -> dict:
    """The planner's configuration and figures for a workload's pipelined
    call, beside the HIP runtime's view of that kernel (registers, spills,
    LDS, resident workgroups per compute unit)."""
    code = DTYPE_CODE[wl.dtype]
    cfg, info = tdg.tdg_plan(code, wl.M, wl.N, wl.K)
    out = {"config": cfg, "plan": info, "resources": None}
    for i in range(tdg.tdg_config_count(code)):
        if tdg.tdg_config_at(code, i) == cfg:
            out["resources"] = tdg.tdg_config_resources(code, i)
            break
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU; this build has no multi-GPU path "
              "(requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import tiled_dense_gemm_loop_amd as tdg
    tdg.load_library()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    wl = si.WORKLOADS[args.workload]
    A, B, dA, dB, C = device_operands(wl)
    run = launcher(tdg, wl, dA, dB, C, "pipelined")
    ms = time_launches(run, args.steps, args.warmup)
    tops, gbs = throughput(wl, ms)
    launches = individual_launches(run)
    cfg, info = tdg.tdg_plan(DTYPE_CODE[wl.dtype], wl.M, wl.N, wl.K)
    unit = UNITS[wl.dtype]
    print("# %s pipelined (%s, %dx%dx%d, %d waves): %.4f ms/launch, %.1f %s"
          % (wl.name, tdg.VARIANT_NAMES[cfg["variant"]], cfg["bm"], cfg["bn"], cfg["bk"],
             cfg["waves"], ms, tops, unit), file=sys.stderr, flush=True)

    table = {}
    if not args.no_table:
        for name, w in si.WORKLOADS.items():
            if name == wl.name:
                a, b, da, db, c = A, B, dA, dB, C
            else:
                a, b, da, db, c = device_operands(w)
            row = {}
            for variant in ("single", "reg_s1", "reg_s2", "direct", "pipelined"):
                t = time_launches(launcher(tdg, w, da, db, c, variant), 100, 20)
                tp, bw = throughput(w, t)
                row[variant] = {"us": round(t * 1e3, 2), "tops": round(tp, 1), "gbs": round(bw, 1)}
            row["speedup_pipelined_vs_single"] = round(row["single"]["us"] / row["pipelined"]["us"], 3)
            if w.M * w.N * w.K <= 1024 ** 3:
                # launch-bound shapes: every form again, replayed from a HIP graph,
                # so that the comparison is between kernels, not host calls
                graph = {}
                for variant in ("single", "reg_s1", "reg_s2", "direct", "pipelined"):
                    t = graph_launches(launcher(tdg, w, da, db, c, variant))
                    tp, bw = throughput(w, t)
                    graph[variant] = {"us": round(t * 1e3, 2), "tops": round(tp, 1),
                                      "gbs": round(bw, 1)}
                graph["speedup_pipelined_vs_single"] = round(
                    graph["single"]["us"] / graph["pipelined"]["us"], 3)
                row["graph"] = graph
            table[name] = row
            print("# %-12s %s" % (name, json.dumps(row)), file=sys.stderr, flush=True)
            if name != wl.name:
                del a, b, da, db, c
                torch.cuda.empty_cache()

    sweep = None
    if not args.no_sweep:
        sweep = tile_sweep(tdg, args.sweep_steps, max(1, args.sweep_steps // 5))
        for r in sweep:
            print("# sweep fp16 4096^3 %s" % json.dumps(r), file=sys.stderr, flush=True)

    cold = None if args.no_table else cold_launches(tdg, si.WORKLOADS["fp16_skinny"])
    if cold:
        print("# cold (512 MiB scrub before each launch) %s" % json.dumps(cold), file=sys.stderr,
              flush=True)
    ladder = None if args.no_ladder else transpose_ladder(tdg)
    ceilings = {} if args.no_ceilings else measured_ceilings(tdg, ladder)

    if args.copy_calib_mib:
        n = args.copy_calib_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    PART_NAMES = ("fp16_4096", "int8_4096", "fp16_skinny")
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, A, B, args.cpu_seconds, args.part_cpu_seconds,
                           ("int8_256", "fp16_1024") + PART_NAMES)

    kernel_desc = "%dx%dx%d tile, %d waves, %d LDS stages, %s" % (
        cfg["bm"], cfg["bn"], cfg["bk"], cfg["waves"], cfg["lds_stages"],
        tdg.VARIANT_NAMES[cfg["variant"]])
    traffic = profiled_traffic(wl.name, kernel_desc)
    alg_bytes = (wl.M * wl.K + wl.K * wl.N) * ELEM_BYTES[wl.dtype] + wl.M * wl.N * 4
    bound = roofline_bound(2.0 * wl.M * wl.N * wl.K, alg_bytes, PEAK[wl.dtype] * 1e3,
                           HBM_PEAK_GBS)
    if bound == "mfma":
        achieved, peak, r_unit = round(tops, 2), PEAK[wl.dtype], unit
        measured = ceilings.get({"f16": "mfma_f16_tflops", "i8": "mfma_i8_tops",
                                 "f32": "mfma_f32_tflops"}[wl.dtype])
    else:
        achieved, peak, r_unit = round(gbs, 1), HBM_PEAK_GBS, "GB/s"
        measured = ceilings.get("copy_gbs")
    # The metric has three parts: FP16 and INT8 4096^3 against the dense MFMA
    # peak, and the skinny product against HBM.  `value` is the headline
    # workload's; the three together, each with its fraction of the
    # data-sheet peak (and of the measured ceiling when one was measured) and
    # the oracle's rate on the same workload, go in `metric_parts` and in
    # roofline.parts.  Each part is timed like the headline (args.steps
    # launches after args.warmup).
    parts = None
    if not args.no_parts:
        def part(name, use_gbs, peak_v, unit_v, ceiling_key):
            w = si.WORKLOADS[name]
            if name == wl.name:
                t = ms
            else:
                _, _, da, db, c = device_operands(w)
                t = time_launches(launcher(tdg, w, da, db, c, "pipelined"), args.steps, args.warmup)
                del da, db, c
                torch.cuda.empty_cache()
            tp, bw = throughput(w, t)
            v = round(bw if use_gbs else tp, 1)
            c = ceilings.get(ceiling_key)
            out = {"value": v, "unit": unit_v, "us": round(t * 1e3, 2), "peak": peak_v,
                   "frac": round(v / peak_v, 4)}
            if c:
                out["frac_of_measured"] = round(v / c, 4)
            if cpu:
                out["cpu_oracle_gops"] = cpu["per_config"][name]["value"]
            return out
        parts = {"fp16_4096": part("fp16_4096", False, PEAK["f16"], "TFLOP/s", "mfma_f16_tflops"),
                 "int8_4096": part("int8_4096", False, PEAK["i8"], "TOP/s", "mfma_i8_tops"),
                 "fp16_skinny": part("fp16_skinny", True, HBM_PEAK_GBS, "GB/s", "copy_gbs")}
        print("# metric parts %s" % json.dumps(parts), file=sys.stderr, flush=True)
    roofline = {"bound": bound, "achieved": achieved, "peak": peak,
                "unit": r_unit, "frac": round(achieved / peak, 4), "traffic": traffic}
    if measured:
        roofline["measured_peak"] = measured
        roofline["frac_of_measured"] = round(achieved / measured, 4)
    if parts:
        roofline["parts"] = parts
    # the headline is the roofline's own quantity: operations per second for
    # an MFMA-bound product, bytes per second for an HBM-bound one
    line = {
        "metric": METRIC,
        "value": achieved,
        "unit": r_unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "M": wl.M, "N": wl.N, "K": wl.K,
                   "accumulate": "i32" if wl.dtype == "i8" else "f32",
                   "kernel": kernel_desc,
                   "parallelism": "none"},
        "roofline": roofline,
        "metric_parts": parts,
        "cpu_baseline": cpu,
    }
    # Everything else measured goes to stderr and, when asked, to a file: the
    # one stdout line stays short enough to be read whole.
    detail = {"line": line, "measured_ceilings": ceilings, "launches": launches, "cold": cold,
              "variants": table or None, "transpose_ladder": ladder, "tile_sweep": sweep,
              "kernels": {name: kernel_record(tdg, si.WORKLOADS[name])
                          for name in PART_NAMES + ("int8_256", "fp16_1024", "fp32_4096")}}
    if args.detail_out:
        d = os.path.dirname(os.path.abspath(args.detail_out))
        os.makedirs(d, exist_ok=True)
        with open(args.detail_out, "w") as f:
            json.dump(detail, f, indent=1)
    print("# launches %s" % json.dumps(launches), file=sys.stderr, flush=True)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
