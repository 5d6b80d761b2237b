"""Measure the planner's kernel-time table and print it as C++.

The planner picks, among the built direct-to-LDS configurations with a
128-byte K tile, the one with the least predicted kernel time.  Its data is
T(n, K) = a(n) + b(n) * K microseconds for n workgroups, measured here at
K = 1024 and K = 4096 on one MI355X: n tiles laid out close to square
(tiles_m x tiles_n from GRIDS), each point timed as HIP-graph replays (FP16,
INT8) or back-to-back launches (FP32, whose kernels are long enough).  Each
series is made non-decreasing in n (a later point caps the earlier ones:
more workgroups cannot finish sooner), and (a, b) follow from the two K.  A
fitted intercept below zero (the K = 1024 time is less than a quarter of the
K = 4096 one) is clamped to zero, keeping the K = 4096 point: no launch
costs less than nothing.  Given several measurement files (several boxes),
emit averages them point by point before fitting.

    python -m tiled_dense_gemm_loop_amd.tune_planner measure times.json   # GPU
    python -m tiled_dense_gemm_loop_amd.tune_planner emit times.json [more.json ...]

The emitted rows replace kPerf in csrc/tdg_api.hip.
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

GRIDS = [(4, 8), (8, 8), (8, 16), (12, 16), (16, 16), (16, 20), (16, 24), (16, 32), (24, 32),
         (32, 32), (32, 48), (48, 48)]
KS = (1024, 4096)
DTYPES = (("f16", 0, 2), ("i8", 1, 1), ("f32", 2, 4))
# preference order inside a 3% tie: the table order below
ORDER = [(256, 256, 8, 2), (256, 256, 4, 2), (256, 128, 4, 2), (256, 128, 4, 3), (128, 128, 4, 4),
         (128, 128, 4, 2), (128, 128, 4, 3), (128, 64, 4, 4), (128, 64, 4, 2), (128, 64, 4, 6),
         (64, 64, 4, 4), (64, 64, 4, 2), (64, 64, 4, 8)]


def measure(path):
    import torch
    import tiled_dense_gemm_loop_amd as tdg
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    from bench import graph_launches, time_launches  # the timing helpers of bench.py
    tdg.load_library()
    out = {}
    for K in KS:
        for dt, code, es in DTYPES:
            side = GRIDS[-1][1] * 256
            if dt == "f16":
                A = torch.randn(side, K, device="cuda").half()
                B = torch.randn(K, side, device="cuda").half()
                C = torch.empty(side, side, device="cuda")
                fex = tdg.gemm_f16f32_ex
            elif dt == "i8":
                A = torch.randint(-128, 128, (side, K), device="cuda", dtype=torch.int8)
                B = torch.randint(-128, 128, (K, side), device="cuda", dtype=torch.int8)
                C = torch.empty(side, side, device="cuda", dtype=torch.int32)
                fex = tdg.gemm_i8i32_ex
            else:
                A = torch.randn(side, K, device="cuda")
                B = torch.randn(K, side, device="cuda")
                C = torch.empty(side, side, device="cuda")
                fex = tdg.gemm_f32f32_ex
            for i in range(tdg.tdg_config_count(code)):
                cf = tdg.tdg_config_at(code, i)
                if cf["variant"] != tdg.TDG_VARIANT_DIRECT_LDS or cf["bk"] * es != 128:
                    continue
                key = "%s %dx%d w%d s%d" % (dt, cf["bm"], cf["bn"], cf["waves"], cf["lds_stages"])
                row = []
                for tm, tn in GRIDS:
                    M, N = tm * cf["bm"], tn * cf["bn"]
                    a, b, c = A[:M], B[:, :N], C[:M, :N]
                    run = lambda: fex(a, b, c, cfg=cf)
                    ms = (time_launches(run, 6, 2) if dt == "f32"
                          else graph_launches(run, per_graph=10, replays=5))
                    row.append([tm * tn, round(ms * 1e3, 2)])
                out.setdefault(str(K), {})[key] = row
                print(K, key, row, flush=True)
            del A, B, C
            torch.cuda.empty_cache()
    json.dump(out, open(path, "w"))


def fit_row(t1, t4):
    """(a, b) of T = a + b * K through the K = 1024 and K = 4096 series,
    with negative intercepts clamped to zero (the K = 4096 point kept)."""
    a_out, b_out = [], []
    for x, y in zip(t1, t4):
        b = (y - x) / (KS[1] - KS[0])
        a = x - KS[0] * b
        if a < 0.0:
            a, b = 0.0, y / KS[1]
        a_out.append(a)
        b_out.append(max(b, 0.0))
    return a_out, b_out


def emit(*paths):
    datas = [json.load(open(p)) for p in paths]

    def mean_series(k, key):
        per = [d[str(k)][key] for d in datas if key in d.get(str(k), {})]
        return [sum(r[i][1] for r in per) / len(per) for i in range(len(per[0]))]
    ns = [tm * tn for tm, tn in GRIDS]
    print("const int kPerfN[%d] = {%s};" % (len(ns), ", ".join(str(n) for n in ns)))
    print("const PerfRow kPerf[] = {")
    for dt, code, _ in DTYPES:
        for bm, bn, w, s in ORDER:
            key = "%s %dx%d w%d s%d" % (dt, bm, bn, w, s)
            if not all(key in d.get(str(KS[1]), {}) for d in datas):
                continue

            def series(k):
                t = mean_series(k, key)
                for i in range(len(t) - 2, -1, -1):   # more workgroups never finish sooner
                    t[i] = min(t[i], t[i + 1])
                return t
            a, b = fit_row(series(KS[0]), series(KS[1]))
            print("    {%d, %d, %d, %d, %d, {%s},\n     {%s}}," % (
                code, bm, bn, w, s, ", ".join("%.2ff" % v for v in a),
                ", ".join("%.6ff" % v for v in b)))
    print("};")


if __name__ == "__main__":
    if sys.argv[1] == "measure":
        measure(sys.argv[2])
    else:
        emit(*sys.argv[2:])
