"""Write the bottleneck report of each benchmarked workload.

The report follows the layout of "Analyze Kernel Bottleneck", Step 8
(baseline, roofline classification, occupancy, compute/load ratio,
instruction mix, LDS cliff, ranked recommendations), with gfx950 in place
of the page's GPU: the LDS is 160 KiB per compute unit, the instruction mix
comes from rocprofv3's SQ instruction counters (no binary is taken apart),
and the recommendations come from the decision matrix of Step 7 applied to
what was measured.

Inputs, and nothing else:
  * the detail file a benchmark run writes (``bench.py --detail-out F``):
    the JSON line, the measured ceilings, and each workload's planned
    configuration beside the runtime's register / LDS / occupancy figures;
  * the rocprofv3 summaries ``profiles/gemm_<workload>_*.md`` (kernel trace,
    HBM traffic, L2 hits, MFMA / LDS counters, instruction counts).

    python -m tiled_dense_gemm_loop_amd.report DETAIL.json [profiles_dir]

writes ``profiles/report_<workload>.md`` for the metric's three workloads,
FP32 4096^3, and the two small configurations (INT8 256^3, FP16 1024^3),
which sit far above both roofline floors and are classified as
latency-bound.
"""
from __future__ import annotations

import glob
import json
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

WORKLOADS = {
    # name: (dtype, M, N, K, element bytes, peak, unit, MFMA operations per clock per CU)
    "fp16_4096": ("FP16 -> FP32", 4096, 4096, 4096, 2, 2500.0, "TFLOP/s", 4096),
    "int8_4096": ("INT8 -> INT32", 4096, 4096, 4096, 1, 5000.0, "TOP/s", 8192),
    "fp16_skinny": ("FP16 -> FP32", 16384, 64, 8192, 2, 2500.0, "TFLOP/s", 4096),
    "int8_256": ("INT8 -> INT32", 256, 256, 256, 1, 5000.0, "TOP/s", 8192),
    "fp16_1024": ("FP16 -> FP32", 1024, 1024, 1024, 2, 2500.0, "TFLOP/s", 4096),
    "fp32_4096": ("FP32 -> FP32", 4096, 4096, 4096, 4, 157.3, "TFLOP/s", 256),
}
# The measured MFMA-only ceiling of each compute-bound workload's instruction.
CEILING_KEY = {"fp16_4096": "mfma_f16_tflops", "int8_4096": "mfma_i8_tops", "fp32_4096": "mfma_f32_tflops"}
# A product whose time exceeds both roofline floors by this factor is bound
# by neither: launch, latency, or too little work per compute unit.
LATENCY_FACTOR = 3.0
HBM_GBS = 8000.0
LDS_PER_CU = 160 * 1024
REGS_PER_LANE = 512          # unified VGPR + AGPR file per SIMD lane
SIMDS = 4
WAVE_SLOTS_PER_SIMD = 8
NUM_CU = 256
CLOCK_GHZ = 2.4


def _num(pattern: str, text: str, default=None):
    m = re.search(pattern, text)
    return float(m.group(1)) if m else default


def read_profile(profiles: str, wl: str) -> dict:
    """The figures of one rocprofv3 summary (profiles/gemm_<wl>_*.md)."""
    paths = [p for p in glob.glob(os.path.join(profiles, "gemm_%s_*.md" % wl)) if "sweep" not in p]
    if not paths:
        return {}
    text = open(paths[0]).read()
    out = {"file": os.path.basename(paths[0])}
    m = re.search(r"\| timed \(dispatches \d+\.\.\d+\) \| (\d+) \| ([\d.]+) us", text)
    if m:
        out["kernel_us"] = float(m.group(2))
    for key, pat in (("traffic", r"traffic_bytes: ([\d.]+)"), ("l2_hit", r"l2_hit_rate: ([\d.]+)"),
                     ("mfma_util", r"mfma_util: ([\d.]+)"),
                     ("counted_mfma_per_load", r"counted_mfma_per_load: ([\d.]+)"),
                     ("refetch", r"Fetched ([\d.]+)x the algorithmic"),
                     ("grbm", r"- GRBM_GUI_ACTIVE: ([\d.]+)"), ("waves", r"- SQ_WAVES: ([\d.]+)"),
                     ("vmem_rd", r"- SQ_INSTS_VMEM_RD: ([\d.]+)"), ("vmem_wr", r"- SQ_INSTS_VMEM_WR: ([\d.]+)"),
                     ("lds", r"- SQ_INSTS_LDS: ([\d.]+)"), ("valu", r"- SQ_INSTS_VALU: ([\d.]+)"),
                     ("salu", r"- SQ_INSTS_SALU: ([\d.]+)"), ("bank_conflict", r"- SQ_LDS_BANK_CONFLICT: ([\d.]+)"),
                     ("lds_active", r"- SQ_LDS_IDX_ACTIVE: ([\d.]+)"), ("line_frac", r"line_frac: ([\d.]+)"),
                     ("kernel_frac", r"kernel_frac: ([\d.]+)")):
        v = _num(pat, text)
        if v is not None:
            out[key] = v
    m = re.search(r"- SQ_INSTS_VALU_MFMA_(F16|I8|F32): ([\d.]+)", text)
    if m:
        out["mfma"] = float(m.group(2))
    out["source_sha"] = (re.search(r"Kernel source sha256\[:16\]: (\w+)", text) or [None, None])[1]
    return out


def occupancy(cfg: dict, res: dict, plan: dict) -> list:
    """Rows of the occupancy table: (resource, per workgroup, limit per CU,
    workgroups per CU)."""
    waves = cfg["waves"]
    threads = waves * 64
    rows = []
    if res:
        regs = res["vgprs"]
        per_simd_waves = max(1, -(-waves // SIMDS))
        by_regs = (REGS_PER_LANE // max(1, regs)) // per_simd_waves
        rows.append(("registers", "%d per lane x %d threads" % (regs, threads),
                     "%d per lane per SIMD, %d SIMDs" % (REGS_PER_LANE, SIMDS), by_regs))
        lds = res["lds_bytes"]
    else:
        lds = plan["lds_bytes"]
    rows.append(("LDS", "%.1f KiB" % (lds / 1024.0), "160 KiB (cliffs: >80 KiB 1, >53.3 2, >40 3, >32 4)",
                 LDS_PER_CU // max(1, lds)))
    rows.append(("wave slots", "%d waves" % waves, "%d (%d per SIMD)" % (SIMDS * WAVE_SLOTS_PER_SIMD, WAVE_SLOTS_PER_SIMD),
                 SIMDS * WAVE_SLOTS_PER_SIMD // waves))
    return rows


def recommendations(wl: str, line: dict, part: dict, kern: dict, prof: dict, ceilings: dict) -> list:
    """Step 7's decision matrix on the measured figures, ranked by the gain
    each could at most bring (its share of the time)."""
    dtype, M, N, K, es, peak, unit, ops_clk = WORKLOADS[wl]
    plan = kern["plan"]
    recs = []
    us = prof.get("kernel_us") or part["us"]
    alg = (M * K + K * N) * es + M * N * 4
    if 2.0 * M * N * K / alg < peak * 1000.0 / HBM_GBS:   # below the balance point: memory side
        copy = ceilings.get("copy_gbs")
        gbs = alg / (us * 1e-6) / 1e9
        gain = max(0.0, 1.0 - gbs / HBM_GBS)
        recs.append((gain, "HBM stream: %.0f GB/s, %.0f%% of the %.0f GB/s data-sheet rate%s.  The product reads "
                           "%.0f times what it writes, and reads stream faster than a copy's mix.  Keep enough bytes "
                           "in flight per CU (the deeper LDS ring) and spread the rows' K walks over the HBM "
                           "channels; at most %.0f%% left to the data-sheet rate." % (
                               gbs, 100 * gbs / HBM_GBS, HBM_GBS,
                               (" and %.0f%% of this box's copy kernel (%.0f GB/s, reading and writing)" % (100 * gbs / copy, copy)) if copy else "",
                               ((M * K + K * N) * es) / (M * N * 4.0), 100 * gain)))
        recs.append((0.0, "Tile reuse cannot help an HBM-bound product with N = %d: A is read once already "
                          "(fetched %.2fx A + B)." % (N, prof.get("refetch", float("nan")))))
        return sorted(recs, key=lambda r: -r[0])
    # compute side
    ceiling_key = CEILING_KEY.get(wl)
    ceil = ceilings.get(ceiling_key) if ceiling_key else None
    achieved = 2.0 * M * N * K / (us * 1e-6) / 1e12
    util = prof.get("mfma_util")
    grbm = prof.get("grbm")
    if grbm and prof.get("vmem_rd"):
        cycles = grbm / 8.0                    # per XCD: the dispatch's active cycles
        fill = prof["vmem_rd"] * 1024.0 / NUM_CU / cycles
        need = plan["need_bytes_per_clk"]
        gain = max(0.0, 1.0 - fill / need) if util is None else max(0.0, min(1.0 - util, 1.0 - fill / need))
        recs.append((gain, "L2 -> LDS fill: averaged over the launch, the tile stream moves %.1f B per clock per "
                           "CU (counted 16-byte wave loads over the active cycles) against the %.0f B the %dx%d "
                           "tile needs at the full MFMA rate; L2 hit rate %.1f%%, A + B fetched %.2fx.  The average "
                           "includes the prologue and the C write, when no tile is copied, and the fill's share "
                           "cannot exceed the cycles the matrix cores are idle, so %.0f%% is a bound, not an "
                           "estimate.  More operations per byte per CU (a larger tile) would lower the need." % (
                               fill, need, kern["config"]["bm"], kern["config"]["bn"], 100 * prof.get("l2_hit", 0),
                               prof.get("refetch", float("nan")), 100 * gain)))
    c_share = M * N * 4 / (prof.get("traffic") or alg)
    t_c = M * N * 4 / (HBM_GBS * 1e3)          # us at the data-sheet write rate
    recs.append((t_c / us, "C write: %d MB of %s output (%.0f%% of the traffic) is written after the last K tile "
                           "by every workgroup at once, with no MFMA work left to overlap it: about %.1f us at "
                           "HBM's data-sheet rate, %.0f%% of the kernel." % (M * N * 4 / 1e6, "INT32" if es == 1 else "FP32",
                                                                               100 * c_share, t_c, 100 * t_c / us)))
    if ceil:
        gain = max(0.0, 1.0 - achieved / ceil)
        recs.append((gain * 0.5, "Clock: the MFMA-only probe sustains %.0f %s on this box with random operands, "
                                 "%.0f%% of the dense peak, i.e. about %.2f GHz of the %.1f GHz the peak assumes "
                                 "(the power limit); the GEMM reaches %.0f%% of it.  Fewer bytes moved per "
                                 "operation (LDS reads, L2 traffic) leave more of the power budget to the matrix "
                                 "cores." % (ceil, unit, 100 * ceil / peak, CLOCK_GHZ * ceil / peak, CLOCK_GHZ,
                                             100 * achieved / ceil)))
    if kern["config"]["variant"] != 3:
        recs.append((0.05, "Use the direct-to-LDS loop: the register-prefetch loop's drain costs LDS write "
                           "bandwidth and registers."))
    return sorted(recs, key=lambda r: -r[0])


def latency_recommendations(wl: str, us: float, call_us, kern: dict, prof: dict) -> list:
    """What holds a product that sits far above both roofline floors, ranked
    by the share of time each could at most recover."""
    dtype, M, N, K, es, peak, unit, ops_clk = WORKLOADS[wl]
    cfg, plan = kern["config"], kern["plan"]
    recs = []
    grid = plan["grid"]
    per_wg = (cfg["bm"] + cfg["bn"]) * K * es
    # the shorter of the trace's kernel time and the graph-replayed launch
    kus = min(prof.get("kernel_us") or us, us)
    rate = per_wg / (kus * 1e-6) / (CLOCK_GHZ * 1e9)
    if grid < NUM_CU:
        recs.append((1.0 - grid / float(NUM_CU),
                     "Compute units: %d workgroups of %dx%d for %d CUs, so %.0f%% of the chip works.  K = %d is "
                     "%d K tile(s), too few to split over more workgroups (split K keeps at least two K tiles "
                     "per part); the product is as wide as its tiles allow." % (
                         grid, cfg["bm"], cfg["bn"], NUM_CU, 100.0 * grid / NUM_CU, K, plan["num_tiles"])))
    else:
        recs.append((1.0 - min(1.0, rate / plan["need_bytes_per_clk"]),
                     "L2 -> LDS fill per CU: each workgroup copies %.0f KiB (its A and B panels), %.1f B per "
                     "clock at %.1f GHz over %.2f us, against the %.0f B per clock a %dx%d tile "
                     "needs to keep the matrix cores busy.  %d workgroups fill the %d CUs once, and no tile "
                     "gives every CU work with fewer bytes; split K over larger tiles halves the bytes per CU "
                     "but adds a summation pass (gemm_*_splitk, when its plan predicts a gain)." % (
                         per_wg / 1024.0, rate, CLOCK_GHZ, kus, plan["need_bytes_per_clk"], cfg["bm"], cfg["bn"],
                         grid, NUM_CU)))
    if call_us and call_us > us:
        recs.append(((call_us - us) / call_us,
                     "Launch: a call through the Python binding takes %.2f us against %.2f us per launch replayed "
                     "from a HIP graph; the difference is host time per call.  Capture repeated calls in a graph "
                     "(the library records into a capturing stream like any HIP call)." % (call_us, us)))
    floor = 2.0 * M * N * K / (peak * 1e12) * 1e6
    recs.append((0.0, "The matrix cores' share is %.2f us of the %.2f us (%.0f%%): nothing on the MFMA side is "
                      "worth changing at this size." % (floor, us, 100.0 * floor / us)))
    return sorted(recs, key=lambda r: -r[0])


def report(wl: str, detail: dict, profiles: str) -> str:
    dtype, M, N, K, es, peak, unit, ops_clk = WORKLOADS[wl]
    line = detail["line"]
    part = (line.get("metric_parts") or {}).get(wl) or {}
    call_us = None
    var = (detail.get("variants") or {}).get(wl) or {}
    if not part and var.get("graph", {}).get("pipelined"):
        # the small configurations: kernel-bound time from HIP-graph replays
        part = {"us": var["graph"]["pipelined"]["us"]}
        call_us = (var.get("pipelined") or {}).get("us")
    elif not part and var.get("pipelined"):
        # a long product outside the metric: its back-to-back launches
        part = {"us": var["pipelined"]["us"]}
    kern = detail["kernels"][wl]
    cfg, plan, res = kern["config"], kern["plan"], kern.get("resources")
    prof = read_profile(profiles, wl)
    ceilings = detail.get("measured_ceilings") or {}
    ops = 2.0 * M * N * K
    alg = (M * K + K * N) * es + M * N * 4
    ai = ops / alg
    balance = peak * 1000.0 / HBM_GBS
    us = part.get("us")
    kus = prof.get("kernel_us")
    variant = {1: "sequential", 2: "register prefetch", 3: "direct-to-LDS"}[cfg["variant"]]
    name = "%s %dx%dx%d, %dx%dx%d tile, %d waves, %d LDS buffers, %s" % (
        dtype, M, N, K, cfg["bm"], cfg["bn"], cfg["bk"], cfg["waves"], cfg["lds_stages"], variant)
    L = ["# Bottleneck report: %s" % wl, "",
         "Kernel: %s." % name,
         "Inputs: the benchmark's detail file (%s; %d timed launches after %d) and `profiles/%s`." % (
             "this run", line["steps"], line["warmup"], prof.get("file", "(no profile)")), ""]
    # Baseline
    L += ["## Baseline", "",
          "- Problem: M = %d, N = %d, K = %d, %s; %d operations, %d algorithmic bytes (A and B read once, C written once)." % (
              M, N, K, dtype, ops, alg)]
    if us and call_us is None:
        L.append("- Time per launch (HIP events, back-to-back launches): %.2f us -> %.1f %s, %.1f GB/s algorithmic." % (
            us, ops / (us * 1e-6) / 1e12, unit, alg / (us * 1e-6) / 1e9))
    elif us:
        L.append("- Time per launch replayed from HIP graphs (20 launches per graph): %.2f us -> %.1f %s, %.1f GB/s "
                 "algorithmic." % (us, ops / (us * 1e-6) / 1e12, unit, alg / (us * 1e-6) / 1e9))
        if call_us:
            L.append("- Time per call through the binding (HIP events, back-to-back calls): %.2f us." % call_us)
    if kus:
        L.append("- Kernel time in the rocprofv3 trace of the timed launches: %.2f us -> %.1f %s." % (
            kus, ops / (kus * 1e-6) / 1e12, unit))
    # Roofline
    bound = "memory" if ai < balance else "compute"
    t_mfma, t_hbm = ops / (peak * 1e12) * 1e6, alg / (HBM_GBS * 1e9) * 1e6
    if us and us > LATENCY_FACTOR * max(t_mfma, t_hbm):
        bound = "latency"
    L += ["", "## Roofline classification", "",
          "- Arithmetic intensity: %.1f operations per byte (unique bytes); balance point %.1f (%.0f %s dense / %.0f GB/s)." % (
              ai, balance, peak, unit, HBM_GBS),
          "- Classification: **%s-bound**." % bound]
    if bound == "latency":
        L.append("- Floors: %.2f us at the dense peak, %.2f us at HBM's rate; the launch takes %.2f us, %.0fx the "
                 "larger.  Neither roofline applies: %.1f%% of the %s peak, %.1f%% of HBM." % (
                     t_mfma, t_hbm, us, us / max(t_mfma, t_hbm), 100 * t_mfma / us, unit, 100 * t_hbm / us))
    elif us:
        if bound == "compute":
            att = ops / (us * 1e-6) / 1e12 / peak
            L.append("- Attained: %.1f%% of the %.0f %s dense peak." % (100 * att, peak, unit))
            ck = CEILING_KEY.get(wl)
            if ck and ceilings.get(ck):
                L.append("- Against the measured MFMA-only ceiling of this box (%.0f %s): %.1f%%." % (
                    ceilings[ck], unit, 100 * ops / (us * 1e-6) / 1e12 / ceilings[ck]))
        else:
            g = alg / (us * 1e-6) / 1e9
            L.append("- Attained: %.1f%% of %.0f GB/s HBM." % (100 * g / HBM_GBS, HBM_GBS))
            if ceilings.get("copy_gbs"):
                L.append("- Against the copy kernel's %.0f GB/s on this box: %.1f%%." % (
                    ceilings["copy_gbs"], 100 * g / ceilings["copy_gbs"]))
    if prof.get("traffic"):
        L.append("- Counted HBM-side traffic: %.1f MB per launch (%.2fx the algorithmic bytes); L2 hit rate %.1f%%." % (
            prof["traffic"] / 1e6, prof["traffic"] / alg, 100 * prof.get("l2_hit", 0.0)))
    # Occupancy
    L += ["", "## Occupancy", "", "| resource | per workgroup | limit per CU | workgroups per CU |",
          "|---|---|---|---|"]
    rows = occupancy(cfg, res, plan)
    for r in rows:
        L.append("| %s | %s | %s | %d |" % r)
    lim = min(r[3] for r in rows)
    limiting = [r[0] for r in rows if r[3] == lim]
    L.append("| **limiting** | | | **%d** (%s) |" % (lim, ", ".join(limiting)))
    if res:
        L.append("")
        L.append("- Runtime occupancy (hipOccupancyMaxActiveBlocksPerMultiprocessor): %d workgroup(s) per CU, "
                 "%d waves per CU, %d per SIMD; planner's estimate %d." % (
                     res["wg_per_cu"], res["wg_per_cu"] * cfg["waves"], res["wg_per_cu"] * cfg["waves"] // SIMDS,
                     plan["wg_per_cu"]))
        L.append("- Registers %d per lane, %d bytes of spills." % (res["vgprs"], res["spill_bytes"]))
    grid = plan["grid"]
    L.append("- Grid: %d workgroups for %d CUs (%.2f rounds)." % (grid, NUM_CU, grid / float(NUM_CU * max(1, lim))))
    # Compute / load ratio
    band = {0: "low (< 5)", 1: "medium (5-20)", 2: "high (> 20)"}[plan["band"]]
    L += ["", "## Compute / load ratio", "",
          "- Per K tile: 2 x %d x %d x %d operations over (%d x %d + %d x %d) x %d bytes = %.1f operations per byte: band %s." % (
              cfg["bm"], cfg["bn"], cfg["bk"], cfg["bm"], cfg["bk"], cfg["bk"], cfg["bn"], es, plan["ratio"], band),
          "- MFMA instructions per 16-byte wave load: %.2f computed from the tile; %s counted (SQ_INSTS_VALU_MFMA over "
          "SQ_INSTS_VMEM_RD, prologue and the loop's repeat load included)." % (
              plan["mfma_per_load"], ("%.2f" % prof["counted_mfma_per_load"]) if "counted_mfma_per_load" in prof else "not"),
          "- At the MFMA rate (%d operations per clock per CU) the tile needs %.1f bytes per clock per CU from L2." % (
              ops_clk, plan["need_bytes_per_clk"]),
          "- Recommendation: the band says %s; on gfx950 the deciding figure is the bytes per clock: at %.0f the copy "
          "has to be hidden, so the pipelined loop (direct-to-LDS: no staging registers, no drain) is used." % (
              "pipelining is probably not worth it" if plan["band"] == 2 else "pipeline", plan["need_bytes_per_clk"])]
    # Instruction mix
    if prof.get("waves"):
        w = prof["waves"]
        L += ["", "## Instruction mix (rocprofv3 SQ instruction counters, per wave)", "",
              "| instruction | count per wave | note |", "|---|---|---|"]
        mfma_note = ("four 32x32x2 MFMAs per 32x32 block per K step of 32 bytes" if es == 4
                     else "one 32x32 block per K step of 32 bytes")
        lds_note = ("fragment reads (`ds_read_b128` for A, four `ds_read_b32` per B fragment)" if es == 4
                    else "fragment reads (`ds_read_b128`, transposing `ds_read_b64_tr`)")
        if "mfma" in prof:
            L.append("| MFMA | %.0f | %s |" % (prof["mfma"] / w, mfma_note))
        L.append("| vector-memory reads | %.0f | 16-byte LDS DMA (`global_load_lds_dwordx4`) |" % (prof.get("vmem_rd", 0) / w))
        L.append("| vector-memory writes | %.0f | C stores, 4 bytes per lane |" % (prof.get("vmem_wr", 0) / w))
        L.append("| LDS | %.0f | %s |" % (prof.get("lds", 0) / w, lds_note))
        L.append("| VALU (non-MFMA) | %.0f | addresses, selects |" % (prof.get("valu", 0) / w))
        L.append("| SALU | %.0f | loop control, wave-uniform bases |" % (prof.get("salu", 0) / w))
        if prof.get("lds_active"):
            L.append("")
            L.append("- LDS bank conflicts: %.0f cycles over %.0f LDS-active cycles (%.3f)." % (
                prof.get("bank_conflict", 0), prof["lds_active"], prof.get("bank_conflict", 0) / prof["lds_active"]))
        if prof.get("mfma_util") is not None:
            L.append("- MfmaUtil (SQ_VALU_MFMA_BUSY_CYCLES per SIMD over the active cycles): %.1f%%." % (100 * prof["mfma_util"]))
        b128 = ceilings.get("lds_b128_bytes_per_clk")
        if b128 and prof.get("lds") and prof.get("grbm"):
            per_instr = 64 * 16 / b128     # cycles per wave-wide LDS read, from the probe
            busy = prof["lds"] / NUM_CU * per_instr / (prof["grbm"] / 8.0)
            L.append("- LDS issue: the probe (`tdg_lds_probe`) measures %.0f bytes per clock per CU for 16-byte "
                     "reads and %.0f for 8-byte transposing ones, i.e. one wave-wide read every %.1f cycles; the "
                     "%.0f LDS instructions per CU keep the LDS busy %.0f%% of the active cycles, before the "
                     "DMA's writes." % (b128, ceilings.get("lds_b64_tr_b16_bytes_per_clk", float("nan")), per_instr,
                                        prof["lds"] / NUM_CU, 100 * busy))
    # LDS cliff
    lds = (res or {}).get("lds_bytes") or plan["lds_bytes"]
    per_cu = LDS_PER_CU // max(1, lds)
    L += ["", "## LDS cliff", "",
          "- LDS per workgroup: %.1f KiB for %d buffers; 160 KiB per CU gives %d workgroup(s) per CU (%s)." % (
              lds / 1024.0, cfg["lds_stages"], per_cu,
              "above the 80 KiB cliff: one workgroup per CU" if lds > 80 * 1024 else "below the 80 KiB cliff"),
          "- %d workgroup(s) of %d waves per CU: %d waves per SIMD; the rest of the latency is hidden inside each "
          "workgroup (the LDS ring and the interleaved fragment reads)." % (
              min(per_cu, (res or {}).get("wg_per_cu", per_cu)), cfg["waves"],
              max(1, min(per_cu, (res or {}).get("wg_per_cu", per_cu)) * cfg["waves"] // SIMDS))]
    # Recommendations
    L += ["", "## Recommended optimizations (ranked by the share of time each could recover)", ""]
    recs = (latency_recommendations(wl, us, call_us, kern, prof) if bound == "latency"
            else recommendations(wl, line, part or {"us": us}, kern, prof, ceilings))
    for i, (g, text) in enumerate(recs, 1):
        L.append("%d. %s" % (i, text))
    return "\n".join(L) + "\n"


def main(argv):
    if not argv:
        print(__doc__)
        return 2
    detail = json.load(open(argv[0]))
    profiles = argv[1] if len(argv) > 1 else os.path.join(ROOT, "profiles")
    for wl in WORKLOADS:
        if wl not in detail.get("kernels", {}):
            continue
        path = os.path.join(profiles, "report_%s.md" % wl)
        open(path, "w").write(report(wl, detail, profiles))
        print("wrote", path)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
