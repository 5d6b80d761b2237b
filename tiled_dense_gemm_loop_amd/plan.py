"""Print what the planner decides for a product, without a GPU.

    python -m tiled_dense_gemm_loop_amd.plan DTYPE M N K [--lda L --ldb L --misalign BYTES]

DTYPE is f16 (FP16 -> FP32), i8 (INT8 -> INT32) or f32 (FP32 -> FP32).  The
output is the planning arithmetic of "Analyze Kernel Bottleneck" (Steps 2,
3, 4 and 6) and "Pipeline GPU Kernel" (Steps 1 and 2) for the chosen
configuration: tile, waves, LDS ring and loop form; the per-tile
compute/load ratio and its band; the LDS bytes and the workgroups per
compute unit they allow; the L2 -> LDS bytes per clock the tile needs at the
MFMA rate; the grid, the K-loop trip count and the predicted kernel time; and
the split-K choice (part count and workspace) of the gemm_*_splitk entry
points.  With leading dimensions or a base misalignment it also reports the
form (bounds-checked or not) a call on such operands runs.
"""
from __future__ import annotations

import argparse
import sys

DTYPES = {"f16": 0, "i8": 1, "f32": 2}
BANDS = {0: "low (< 5)", 1: "medium (5-20)", 2: "high (> 20)"}


def describe(dtype: str, M: int, N: int, K: int, lda=None, ldb=None, misalign: int = 0) -> str:
    import tiled_dense_gemm_loop_amd as t
    code = DTYPES[dtype]
    cfg, info = t.tdg_plan(code, M, N, K)
    L = ["%s %d x %d x %d" % ({"f16": "FP16 -> FP32", "i8": "INT8 -> INT32", "f32": "FP32 -> FP32"}[dtype],
                                M, N, K)]
    L.append("configuration: %dx%dx%d tile, %d waves, %d LDS buffer(s), %s" % (
        cfg["bm"], cfg["bn"], cfg["bk"], cfg["waves"], cfg["lds_stages"], t.VARIANT_NAMES[cfg["variant"]]))
    L.append("ratio: %.1f operations per byte per tile, band %s" % (info["ratio"], BANDS[info["band"]]))
    L.append("LDS: %.1f KiB per workgroup -> %d workgroup(s) per CU (160 KiB per CU)" % (
        info["lds_bytes"] / 1024.0, info["wg_per_cu"]))
    L.append("L2 -> LDS needed at the MFMA rate: %.1f B per clock per CU" % info["need_bytes_per_clk"])
    L.append("MFMA instructions per 16-byte wave load: %.2f" % info["mfma_per_load"])
    L.append("grid: %d workgroups (%.2f per CU), K loop: %d tile(s), %s%s" % (
        info["grid"], info["grid"] / 256.0, info["num_tiles"],
        "pipelined" if info["pipelined"] else "not pipelined (one K tile)",
        ", K walk rotated per tile row" if info["k_rotated"] else ""))
    try:
        us = t.tdg_predict_us(code, cfg["bm"], cfg["bn"], cfg["waves"], cfg["lds_stages"], M, N, K)
        L.append("predicted kernel time: %.1f us (%.1f %s)" % (
            us, 2.0 * M * N * K / (us * 1e-6) / 1e12 if us > 0 else 0.0, "TOP/s" if dtype == "i8" else "TFLOP/s"))
    except t.TdgError:
        L.append("predicted kernel time: outside the measured table")
    parts, ws = t.tdg_splitk_plan(code, M, N, K)
    L.append("split K: %s" % ("not predicted faster" if parts == 1 else
                              "%d parts, workspace %.1f MiB" % (parts, ws / 2.0 ** 20)))
    if lda is not None or ldb is not None or misalign:
        lda = lda if lda is not None else max(K, 1)
        ldb = ldb if ldb is not None else max(N, 1)
        base = (1 << 40) + misalign
        c2, i2 = t.tdg_plan_operands(code, M, N, K, base, lda, base + (1 << 38), ldb)
        L.append("on operands with lda %d, ldb %d, bases %d bytes off 16: %s, %s, %s" % (
            lda, ldb, misalign % 16, "%dx%dx%d" % (c2["bm"], c2["bn"], c2["bk"]),
            t.VARIANT_NAMES[c2["variant"]], "bounds-checked" if i2["guarded"] else "unchecked"))
    return "\n".join(L) + "\n"


def main(argv) -> int:
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("dtype", choices=sorted(DTYPES))
    p.add_argument("M", type=int)
    p.add_argument("N", type=int)
    p.add_argument("K", type=int)
    p.add_argument("--lda", type=int)
    p.add_argument("--ldb", type=int)
    p.add_argument("--misalign", type=int, default=0, help="bytes the bases of A and B sit past 16-byte alignment")
    a = p.parse_args(argv)
    sys.stdout.write(describe(a.dtype, a.M, a.N, a.K, a.lda, a.ldb, a.misalign))
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
