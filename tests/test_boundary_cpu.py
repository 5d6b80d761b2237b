"""CPU tests of the C-ABI library: it loads without a GPU, exports every
symbol include/tdgemm.h declares, rejects bad arguments before touching the
device, and its planner arithmetic reproduces the pages' worked examples
(tests/golden/pages_worked_examples.json).  No GEMM is computed here."""
import ctypes
import json
import os
import re

import pytest

import tiled_dense_gemm_loop_amd as tdg
from conftest import no_device_only

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_worked_examples.json")))
DT = {"f16": tdg.TDG_DTYPE_F16F32, "i8": tdg.TDG_DTYPE_I8I32}


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "tdgemm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    lib = tdg.load_library()
    declared = _declared_functions()
    assert len(declared) >= 10
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(tdg.EXPORTED) == declared


def test_status_strings():
    assert tdg.tdg_status_string(tdg.TDG_OK) == "ok"
    assert "invalid" in tdg.tdg_status_string(tdg.TDG_ERR_INVALID_ARG)
    assert tdg.tdg_status_string(12345) == "unknown status"


# --- argument validation runs before any HIP call ----------------------------------

BAD_CALLS = [
    ("negative M", (-1, 4, 4, 4096, 4, 8192, 4, 1 << 20, 4)),
    ("negative K", (4, 4, -2, 4096, 4, 8192, 4, 1 << 20, 4)),
    ("lda < K", (4, 4, 8, 4096, 4, 8192, 4, 1 << 20, 4)),
    ("ldb < N", (4, 8, 4, 4096, 4, 8192, 4, 1 << 20, 8)),
    ("ldc < N", (4, 8, 4, 4096, 4, 8192, 8, 1 << 20, 4)),
    ("NULL A", (4, 4, 4, 0, 4, 8192, 4, 1 << 20, 4)),
    ("NULL B", (4, 4, 4, 4096, 4, 0, 4, 1 << 20, 4)),
    ("NULL C", (4, 4, 4, 4096, 4, 8192, 4, 0, 4)),
    ("C overlaps A", (4, 4, 4, 4096, 4, 1 << 20, 4, 4096 + 8, 4)),
    ("C overlaps B", (4, 4, 4, 1 << 20, 4, 8192, 4, 8192 - 16, 4)),
    ("M too large", (1 << 31, 4, 4, 4096, 4, 8192, 4, 1 << 40, 4)),
    # sizes keep a 2^16 margin below 2^31 (tile start + extent in 32 bits)
    ("M past the margin", ((1 << 31) - (1 << 16) + 1, 4, 4, 4096, 4, 8192, 4, 1 << 40, 4)),
    ("N past the margin", (4, (1 << 31) - 1, 4, 4096, 4, 1 << 36, (1 << 31) - 1, 1 << 40, (1 << 31) - 1)),
    ("K past the margin", (4, 4, (1 << 31) - 100, 4096, (1 << 31) - 100, 1 << 36, 4, 1 << 40, 4)),
    # rows x leading dimension past int64: no such matrix can exist
    ("lda overflows", (4, 4, 4, 4096, 1 << 62, 1 << 40, 4, 1 << 44, 4)),
    ("ldb overflows", (4, 4, 4, 4096, 4, 1 << 40, 1 << 62, 1 << 44, 4)),
    ("ldc overflows", (4, 4, 4, 4096, 4, 1 << 40, 4, 1 << 44, 1 << 62)),
]


@pytest.mark.parametrize("name", ["gemm_f16f32", "gemm_i8i32", "gemm_f16f32_pipelined",
                                  "gemm_i8i32_pipelined", "gemm_f16f32_ex", "gemm_i8i32_ex"])
@pytest.mark.parametrize("what,args", BAD_CALLS, ids=[b[0] for b in BAD_CALLS])
def test_invalid_arguments(name, what, args):
    assert tdg.call_raw(name, *args) == tdg.TDG_ERR_INVALID_ARG


def test_empty_output_returns_ok_without_a_device():
    # M == 0 or N == 0: nothing to do, no device needed
    assert tdg.call_raw("gemm_f16f32_pipelined", 0, 4, 4, 0, 4, 8192, 4, 0, 4) == tdg.TDG_OK
    assert tdg.call_raw("gemm_i8i32", 4, 0, 4, 4096, 4, 0, 1, 0, 1) == tdg.TDG_OK


# --- copy / transpose ladder: the same validation rules -------------------------------

def _move(name, *args):
    lib = tdg.load_library()
    return getattr(lib, name)(*args)


MOVE_BAD = [
    ("negative rows", (-1, 4, 4096, 4, 1 << 20, 4)),
    ("ldi < cols", (4, 8, 4096, 4, 1 << 20, 8)),
    ("NULL in", (4, 4, 0, 4, 1 << 20, 4)),
    ("NULL out", (4, 4, 4096, 4, 0, 4)),
    ("out overlaps in", (4, 4, 4096, 4, 4096 + 32, 4)),
    ("rows too large", (1 << 31, 4, 4096, 4, 1 << 40, 4)),
    ("ldi overflows", (4, 4, 4096, 1 << 62, 1 << 40, 4)),
    ("ldo overflows", (4, 4, 4096, 4, 1 << 40, 1 << 62)),
]


@pytest.mark.parametrize("what,args", MOVE_BAD, ids=[b[0] for b in MOVE_BAD])
def test_move_invalid_arguments(what, args):
    assert _move("tdg_copy_f32", *args, None) == tdg.TDG_ERR_INVALID_ARG
    for method in range(6):
        assert _move("tdg_transpose_f32", method, *args, None) == tdg.TDG_ERR_INVALID_ARG


def test_move_output_leading_dimension_rules():
    # copy: ldo >= cols; transpose: out is cols x rows, so ldo >= rows
    assert _move("tdg_copy_f32", 8, 16, 4096, 16, 1 << 20, 8, None) == tdg.TDG_ERR_INVALID_ARG
    assert _move("tdg_transpose_f32", 0, 16, 8, 4096, 8, 1 << 20, 8, None) == \
        tdg.TDG_ERR_INVALID_ARG
    # an unknown method
    assert _move("tdg_transpose_f32", 6, 4, 4, 4096, 4, 1 << 20, 4, None) == tdg.TDG_ERR_INVALID_ARG
    assert _move("tdg_transpose_f32", -1, 4, 4, 4096, 4, 1 << 20, 4, None) == \
        tdg.TDG_ERR_INVALID_ARG


def test_move_empty_matrix_returns_ok_without_a_device():
    assert _move("tdg_copy_f32", 0, 5, 0, 5, 0, 5, None) == tdg.TDG_OK
    assert _move("tdg_transpose_f32", 3, 7, 0, 0, 1, 0, 7, None) == tdg.TDG_OK


def test_mfma_probe_arguments():
    lib = tdg.load_library()
    assert lib.tdg_mfma_probe(7, 4, 4096, None) == tdg.TDG_ERR_INVALID_ARG
    assert lib.tdg_mfma_probe(0, 3, 4096, None) == tdg.TDG_ERR_INVALID_ARG
    assert lib.tdg_mfma_probe(0, 4, None, None) == tdg.TDG_ERR_INVALID_ARG
    assert tdg.tdg_mfma_probe_ops(0, 3) == -1 and tdg.tdg_mfma_probe_ops(3, 4) == -1
    assert tdg.tdg_mfma_probe_ops(2, 4) == 2 * 32 * 32 * 2 * 8 * 4 * 2048
    # 512 workgroups x 4 waves x 8 MFMAs per step; 2*32*32*k operations each
    assert tdg.tdg_mfma_probe_ops(0, 4) == 2 * 32 * 32 * 16 * 8 * 4 * 2048
    assert tdg.tdg_mfma_probe_ops(1, 4) == 2 * tdg.tdg_mfma_probe_ops(0, 4)
    assert tdg.tdg_mfma_probe_sink_floats() == 512 * 256


def _offset_bounds(dtype, cfg):
    """Largest lda and ldb (elements) whose rows a kernel reaches with its
    unsigned 32-bit per-lane offsets: a thread's first chunk lies up to
    R - 1 rows below the tile's first row, R = threads / (16-byte chunks per
    image row), and adds up to one image row of bytes."""
    es = {0: 2, 1: 1, 2: 4}[dtype]
    threads = cfg["waves"] * 64
    a_cpr, b_cpr = cfg["bk"] * es // 16, cfg["bn"] * es // 16
    a_rows, b_rows = threads // a_cpr, threads // b_cpr
    lim = (1 << 32) - 1
    lda = (lim - cfg["bk"] * es) // (a_rows - 1) // es
    ldb = (lim - cfg["bn"] * es) // (b_rows - 1) // es
    return lda, ldb


@no_device_only
@pytest.mark.parametrize("dtype", [0, 1, 2])
def test_leading_dimension_bound_of_every_kernel(dtype):
    """For every built configuration, the largest leading dimensions its
    32-bit per-lane offsets reach are accepted (the call gets as far as the
    device check: TDG_ERR_NO_DEVICE on this host) and one element more is
    refused with TDG_ERR_UNSUPPORTED, for A and for B separately; no call
    launches anything here.  Every kernel accepts 33,818,639 bytes."""
    name = {0: "gemm_f16f32_ex", 1: "gemm_i8i32_ex", 2: "gemm_f32f32_ex"}[dtype]
    es = {0: 2, 1: 1, 2: 4}[dtype]
    A, B, C = 1 << 40, 1 << 44, 1 << 46
    for i in range(tdg.tdg_config_count(dtype)):
        c = tdg.tdg_config_at(dtype, i)
        cfg = tdg.TdgConfig(**c)
        M, N, K = c["bm"], c["bn"], 2 * c["bk"]
        lda, ldb = _offset_bounds(dtype, c)
        assert min(lda, ldb) * es >= 33818639 - es
        ok = tdg.call_raw(name, M, N, K, A, lda, B, ldb, C, N, 0, cfg)
        assert ok == tdg.TDG_ERR_NO_DEVICE, (c, lda, ldb, ok)
        assert tdg.call_raw(name, M, N, K, A, lda + 1, B, ldb, C, N, 0, cfg) == \
            tdg.TDG_ERR_UNSUPPORTED, (c, "lda")
        assert tdg.call_raw(name, M, N, K, A, lda, B, ldb + 1, C, N, 0, cfg) == \
            tdg.TDG_ERR_UNSUPPORTED, (c, "ldb")


@no_device_only
def test_oversized_leading_dimension_is_unsupported():
    # the 64 x 64 tile's 256 threads cover 32 rows of A (K tile of 128
    # bytes): 31 * lda * 2 + 128 bytes must stay below 2^32
    lda = ((1 << 32) - 1 - 128) // 31 // 2 + 1
    assert tdg.call_raw("gemm_f16f32_pipelined", 64, 64, 64, 1 << 30, lda, 1 << 40, 64,
                        1 << 44, 64) == tdg.TDG_ERR_UNSUPPORTED
    assert tdg.call_raw("gemm_f16f32_pipelined", 64, 64, 64, 1 << 30, lda - 1, 1 << 40, 64,
                        1 << 44, 64) == tdg.TDG_ERR_NO_DEVICE
    assert tdg.call_raw("gemm_i8i32", 64, 64, 64, 1 << 30, 64, 1 << 40, 1 << 27,
                        1 << 44, 64) == tdg.TDG_ERR_UNSUPPORTED
    # a single row may have any leading dimension; one whose 64-row offset
    # would wrap a 64-bit product must still be refused, not launched
    for lda in (1 << 57, 1 << 59, (1 << 61) - 1):
        assert tdg.call_raw("gemm_f16f32_pipelined", 1, 64, 64, 1 << 30, lda, 1 << 40, 64,
                            1 << 44, 64) == tdg.TDG_ERR_UNSUPPORTED
    assert tdg.call_raw("gemm_i8i32_pipelined", 64, 1, 64, 1 << 30, 64, 1 << 40, 1 << 56,
                        1 << 32, 1) == tdg.TDG_ERR_UNSUPPORTED


def test_unbuilt_configuration_is_unsupported():
    cfg = tdg.TdgConfig(bm=96, bn=96, bk=0, waves=0, lds_stages=0, variant=0)
    with pytest.raises(tdg.TdgError) as e:
        tdg.tdg_plan(tdg.TDG_DTYPE_F16F32, 4096, 4096, 4096, cfg)
    assert e.value.status == tdg.TDG_ERR_UNSUPPORTED
    cfg = tdg.TdgConfig(bm=0, bn=0, bk=0, waves=0, lds_stages=3, variant=tdg.TDG_VARIANT_SINGLE)
    with pytest.raises(tdg.TdgError):
        tdg.tdg_plan(tdg.TDG_DTYPE_F16F32, 4096, 4096, 4096, cfg)


# --- planner arithmetic pinned to the pages -------------------------------------------

@pytest.mark.parametrize("case", GOLDEN["lds_budget"], ids=lambda c: "%s_%dx%dx%d_s%d" % (
    c["dtype"], c["bm"], c["bn"], c["bk"], c["stages"]))
def test_lds_budget_matches_the_pages(case):
    info = tdg.tdg_tile_figures(DT[case["dtype"]], case["bm"], case["bn"], case["bk"],
                                stages=case["stages"])
    assert info["lds_bytes"] == case["lds_bytes"]


def test_tile_figures_argument_ranges():
    """The tile arithmetic takes any tile up to 65536 on a side (its
    products stay exact) and the sizes every entry point accepts; beyond
    those, and for non-positive tiles or waves outside 1..16, it refuses."""
    F16 = tdg.TDG_DTYPE_F16F32
    lim = (1 << 31) - (1 << 16)
    big = tdg.tdg_tile_figures(F16, 65536, 65536, 65536, waves=16, stages=8, M=lim, N=lim, K=lim)
    assert big["lds_bytes"] == 8 * (65536 * 65536 * 2) * 2 and big["wg_per_cu"] == 0
    assert big["est_regs"] > 512
    for args, kw in (((F16, 65537, 64, 64), {}), ((F16, 64, 65537, 64), {}), ((F16, 64, 64, 65537), {}),
                     ((F16, 0, 64, 64), {}), ((F16, 64, 64, 64), {"waves": 17}),
                     ((F16, 64, 64, 64), {"stages": 9}), ((F16, 64, 64, 64), {"M": lim + 1}),
                     ((F16, 64, 64, 64), {"K": -1})):
        with pytest.raises(tdg.TdgError):
            tdg.tdg_tile_figures(*args, **kw)


def test_doubling_doubles():
    for c in GOLDEN["lds_budget"]:
        one = tdg.tdg_tile_figures(DT[c["dtype"]], c["bm"], c["bn"], c["bk"], stages=1)
        two = tdg.tdg_tile_figures(DT[c["dtype"]], c["bm"], c["bn"], c["bk"], stages=2)
        assert two["lds_bytes"] == 2 * one["lds_bytes"]


@pytest.mark.parametrize("case", GOLDEN["balance_points"], ids=lambda c: str(c["balance"]))
def test_balance_points_match_the_pages(case):
    import bench
    assert round(bench.balance_point(case["peak_gops"], case["bw_gbs"]), 1) == case["balance"]


def test_ratio_formula_and_bands():
    # ratio = 2*BM*BN*BK / ((BM*BK + BK*BN) * sizeof(T)), i.e. BM*BN/(BM+BN) for FP16
    for (bm, bn, bk) in [(256, 256, 64), (128, 64, 32), (16, 16, 16), (8, 8, 8), (3, 5, 7)]:
        f16 = tdg.tdg_tile_figures(tdg.TDG_DTYPE_F16F32, bm, bn, bk)
        i8 = tdg.tdg_tile_figures(tdg.TDG_DTYPE_I8I32, bm, bn, bk)
        assert f16["ratio"] == pytest.approx(2 * bm * bn * bk / ((bm * bk + bk * bn) * 2))
        assert i8["ratio"] == pytest.approx(2 * f16["ratio"])
    bands = {(8, 8, 8): 0, (16, 16, 16): 1, (40, 40, 40): 1, (42, 42, 16): 2, (256, 256, 64): 2}
    for (bm, bn, bk), band in bands.items():
        assert tdg.tdg_tile_figures(tdg.TDG_DTYPE_F16F32, bm, bn, bk)["band"] == band
    # the boundaries themselves: ratio 5 -> band 1, ratio 20 -> band 1
    assert tdg.tdg_tile_figures(tdg.TDG_DTYPE_F16F32, 10, 10, 4)["ratio"] == 5.0
    assert tdg.tdg_tile_figures(tdg.TDG_DTYPE_F16F32, 10, 10, 4)["band"] == 1
    assert tdg.tdg_tile_figures(tdg.TDG_DTYPE_F16F32, 40, 40, 4)["band"] == 1


def test_occupancy_limits_follow_the_160k_lds():
    # 256x256 FP16 with a 64-element K tile: 64 KiB per buffer, two buffers
    # 128 KiB -> one workgroup per CU (its 8 waves also fill the registers)
    two = tdg.tdg_tile_figures(tdg.TDG_DTYPE_F16F32, 256, 256, 64, waves=8, stages=2)
    assert (two["lds_bytes"], two["wg_per_cu"]) == (131072, 1)
    # 128x128x64 FP16: 32 KiB per buffer; two buffers -> LDS allows 2 per CU,
    # one buffer would allow 5 and the registers then decide
    two = tdg.tdg_tile_figures(tdg.TDG_DTYPE_F16F32, 128, 128, 64, waves=4, stages=2)
    one = tdg.tdg_tile_figures(tdg.TDG_DTYPE_F16F32, 128, 128, 64, waves=4, stages=1)
    assert (two["lds_bytes"], two["wg_per_cu"]) == (65536, 2)
    assert 2 < one["wg_per_cu"] <= 5
    # 53.3 KiB is the two-per-CU cliff: 54 KiB per workgroup gives two, not three
    assert tdg.tdg_tile_figures(tdg.TDG_DTYPE_I8I32, 128, 88, 256, stages=1)["wg_per_cu"] == 2


def test_needed_bandwidth_and_instruction_ratio():
    """The planner's MI355X figures: L2->LDS bytes per clock per CU that keep
    the MFMAs busy (MFMA ops/clock/CU over the ratio) and MFMA instructions
    per 16-byte wave load instruction."""
    f16 = tdg.tdg_tile_figures(tdg.TDG_DTYPE_F16F32, 256, 256, 64, 8, 2, 3)
    assert f16["ratio"] == 128.0 and f16["need_bytes_per_clk"] == 32.0
    assert f16["mfma_per_load"] == 256 / 64          # 256 MFMAs, 64 KiB of loads
    i8 = tdg.tdg_tile_figures(tdg.TDG_DTYPE_I8I32, 256, 256, 128, 8, 2, 3)
    assert i8["ratio"] == 256.0 and i8["need_bytes_per_clk"] == 32.0 and i8["mfma_per_load"] == 4.0
    f32 = tdg.tdg_tile_figures(tdg.TDG_DTYPE_F32F32, 256, 256, 32, 8, 2, 3)
    assert f32["ratio"] == 64.0 and f32["need_bytes_per_clk"] == 4.0 and f32["mfma_per_load"] == 16.0
    skinny = tdg.tdg_tile_figures(tdg.TDG_DTYPE_F16F32, 64, 64, 64, 4, 4, 3)
    assert skinny["ratio"] == 32.0 and skinny["need_bytes_per_clk"] == 128.0


def test_one_k_tile_is_not_pipelined():
    cfg, info = tdg.tdg_plan(tdg.TDG_DTYPE_F16F32, 4096, 4096, 4096)
    assert info["pipelined"] == 1
    for K in (1, 64):
        cfg, info = tdg.tdg_plan(tdg.TDG_DTYPE_F16F32, 4096, 4096, K)
        assert cfg["variant"] == tdg.TDG_VARIANT_SINGLE and info["pipelined"] == 0
        assert info["num_tiles"] == 1
    cfg, info = tdg.tdg_plan(tdg.TDG_DTYPE_F16F32, 4096, 4096, 65)
    assert info["num_tiles"] == 2 and info["pipelined"] == 1


def test_grid_and_trip_count():
    info = tdg.tdg_tile_figures(tdg.TDG_DTYPE_F16F32, 256, 256, 64, 8, 2, 3, 4096, 4096, 4100)
    assert info["grid"] == 256 and info["num_tiles"] == 65


def test_planner_choices():
    cfg, info = tdg.tdg_plan(tdg.TDG_DTYPE_F16F32, 4096, 4096, 4096)
    assert (cfg["bm"], cfg["bn"], cfg["variant"]) == (256, 256, tdg.TDG_VARIANT_DIRECT_LDS)
    assert info["grid"] == 256 and info["guarded"] == 0
    cfg, info = tdg.tdg_plan(tdg.TDG_DTYPE_F16F32, 16384, 64, 8192)
    assert cfg["bn"] == 64 and cfg["lds_stages"] >= 2 and info["grid"] >= 256
    # ragged shapes keep the copy in the DMA's bounds-checked form, whether
    # or not N and K are whole 16-byte chunks (dense operands: rows off the
    # 16-byte grid when they are not)
    for code, M, N, K in [(0, 300, 264, 200), (0, 4000, 4000, 4000), (1, 300, 272, 144),
                          (0, 16383, 64, 8192), (1, 1, 16, 272), (1, 300, 290, 333),
                          (0, 300, 264, 201), (0, 300, 260, 200), (1, 300, 272, 136)]:
        cfg, info = tdg.tdg_plan(code, M, N, K)
        assert info["guarded"] == 1 and cfg["variant"] == tdg.TDG_VARIANT_DIRECT_LDS, (M, N, K)
    # one K tile: nothing to overlap, the sequential loop
    cfg, info = tdg.tdg_plan(tdg.TDG_DTYPE_F16F32, 300, 264, 33)
    assert cfg["variant"] == tdg.TDG_VARIANT_SINGLE and info["pipelined"] == 0
    # the 4000^3 plan keeps the 256x256 tile of the 4096^3 one
    cfg, _ = tdg.tdg_plan(tdg.TDG_DTYPE_F16F32, 4000, 4000, 4000)
    assert (cfg["bm"], cfg["bn"]) == (256, 256)
    # FP32 inputs: the same 256 x 256 direct-to-LDS plan at 4096^3
    cfg, info = tdg.tdg_plan(tdg.TDG_DTYPE_F32F32, 4096, 4096, 4096)
    assert (cfg["bm"], cfg["bn"], cfg["variant"]) == (256, 256, tdg.TDG_VARIANT_DIRECT_LDS)
    assert cfg["bk"] == 32 and info["guarded"] == 0 and info["ratio"] == 64.0
    cfg, info = tdg.tdg_plan(tdg.TDG_DTYPE_F32F32, 300, 260, 200)
    assert info["guarded"] == 1 and cfg["variant"] == tdg.TDG_VARIANT_DIRECT_LDS
    cfg, info = tdg.tdg_plan(tdg.TDG_DTYPE_F32F32, 300, 262, 200)
    assert info["guarded"] == 1 and cfg["variant"] == tdg.TDG_VARIANT_DIRECT_LDS
    # every built configuration can be planned back exactly
    for code in (0, 1, 2):
        for i in range(tdg.tdg_config_count(code)):
            c = tdg.tdg_config_at(code, i)
            got, _ = tdg.tdg_plan(code, 4 * c["bm"], 4 * c["bn"], 8 * c["bk"], dict(c))
            assert got == c


def test_debug_flags_round_trip():
    """The race-screen switch is host state: set, read back, reset; unknown
    bits are rejected without changing the setting."""
    assert tdg.tdg_set_debug_flags(tdg.TDG_DEBUG_POISON_LDS) == 0
    with pytest.raises(tdg.TdgError):
        tdg.tdg_set_debug_flags(4)
    assert tdg.tdg_set_debug_flags(0) == tdg.TDG_DEBUG_POISON_LDS
    assert tdg.tdg_set_debug_flags(0) == 0


@no_device_only
def test_concurrent_calls_resolve_consistently():
    """Eight host threads resolve a churn of shapes and explicit configs at
    once through the GEMM entry points (the plan cache holds 16 entries, so
    slots are replaced while others read them).  Every status must equal the
    one a single thread gets: TDG_ERR_NO_DEVICE for a plan that resolves (no
    GPU here; resolution runs first) and TDG_ERR_UNSUPPORTED for a config
    that is not built.  ctypes releases the GIL during each call."""
    import random
    import threading
    bad = tdg.TdgConfig(96, 96, 64, 4, 2, tdg.TDG_VARIANT_DIRECT_LDS)   # not built
    calls = []
    rng = random.Random(3)
    for _ in range(400):
        M, N, K = rng.randint(1, 5000), rng.randint(1, 5000), rng.randint(1, 5000)
        name = rng.choice(["gemm_f16f32_pipelined", "gemm_i8i32", "gemm_f32f32_ex",
                           "gemm_i8i32_ex"])
        cfg = bad if name.endswith("_ex") and rng.random() < 0.5 else (
            tdg.TdgConfig() if name.endswith("_ex") else None)
        # fake, 16-byte aligned, non-overlapping pointers: nothing is dereferenced
        calls.append((name, M, N, K, 1 << 40, K, 2 << 40, N, 3 << 40, N, 0, cfg))
    expected = [tdg.call_raw(*c) for c in calls]
    assert set(expected) <= {tdg.TDG_ERR_NO_DEVICE, tdg.TDG_ERR_UNSUPPORTED}
    assert tdg.TDG_ERR_UNSUPPORTED in expected and tdg.TDG_ERR_NO_DEVICE in expected
    got = [[None] * len(calls) for _ in range(8)]

    def worker(w):
        order = list(range(len(calls)))
        random.Random(w).shuffle(order)
        for _ in range(3):
            for i in order:
                got[w][i] = tdg.call_raw(*calls[i])

    threads = [threading.Thread(target=worker, args=(w,)) for w in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    for w in range(8):
        assert got[w] == expected, "thread %d disagrees" % w


def test_k_rotation_rule():
    """Tile rows walk K from their own offsets exactly when all of B fits in
    2 MiB (half an XCD's L2)."""
    cases = [((tdg.TDG_DTYPE_F16F32, 16384, 64, 8192), 1),      # B = 1 MiB
             ((tdg.TDG_DTYPE_F16F32, 1024, 1024, 1024), 1),     # B = 2 MiB
             ((tdg.TDG_DTYPE_F16F32, 1024, 1024, 1025), 0),
             ((tdg.TDG_DTYPE_F16F32, 4096, 4096, 4096), 0),
             ((tdg.TDG_DTYPE_I8I32, 4096, 4096, 4096), 0),
             ((tdg.TDG_DTYPE_I8I32, 256, 256, 256), 1),
             ((tdg.TDG_DTYPE_F32F32, 4096, 128, 4096), 1),      # B = 2 MiB
             ((tdg.TDG_DTYPE_F32F32, 4096, 129, 4096), 0)]
    for args, want in cases:
        _, info = tdg.tdg_plan(*args)
        assert info["k_rotated"] == want, args


def _plan_str(code, M, N, K, **req):
    cfg, _ = tdg.tdg_plan(code, M, N, K, cfg=req or None)
    return "%dx%d w%d s%d %s" % (cfg["bm"], cfg["bn"], cfg["waves"], cfg["lds_stages"],
                                 tdg.VARIANT_NAMES[cfg["variant"]])


def test_planner_picks_by_predicted_time():
    """The planner minimises the measured-time model over the built direct-
    to-LDS configurations.  Where the older rule (the largest tile that still
    fills all 256 CUs) lost 26-51% on MI355X, it now takes the larger tile
    with fewer workgroups; the benchmark shapes keep their configurations."""
    F16, I8 = tdg.TDG_DTYPE_F16F32, tdg.TDG_DTYPE_I8I32
    assert _plan_str(F16, 4096, 4096, 4096) == "256x256 w8 s2 direct_lds"
    assert _plan_str(I8, 4096, 4096, 4096) == "256x256 w8 s2 direct_lds"
    assert _plan_str(F16, 1024, 1024, 1024) == "64x64 w4 s4 direct_lds"
    assert _plan_str(F16, 16384, 64, 8192) == "64x64 w4 s4 direct_lds"
    assert _plan_str(F16, 4000, 4000, 4000) == "256x256 w8 s2 direct_lds"
    # 144 and 196 workgroups of 256 x 256 beat 288 and 392 of 256 x 128
    assert _plan_str(F16, 3072, 3072, 3072) == "256x256 w8 s2 direct_lds"
    assert _plan_str(F16, 3584, 3584, 3584) == "256x256 w8 s2 direct_lds"
    # 144 workgroups of 128 x 128 beat 288 of 128 x 64
    assert _plan_str(F16, 1536, 1536, 1536) == "128x128 w4 s4 direct_lds"
    assert _plan_str(I8, 2560, 2560, 2560) == "128x128 w4 s2 direct_lds"


def _perf_rows(dtype):
    """(bm, bn, waves, stages) of every row of the measured-time table."""
    rows = []
    for i in range(tdg.tdg_config_count(dtype)):
        c = tdg.tdg_config_at(dtype, i)
        es = {0: 2, 1: 1, 2: 4}[dtype]
        if c["variant"] != tdg.TDG_VARIANT_DIRECT_LDS or c["bk"] * es != 128:
            continue
        key = (c["bm"], c["bn"], c["waves"], c["lds_stages"])
        try:
            tdg.tdg_predict_us(dtype, *key, 256, 256, 256)
        except tdg.TdgError:
            continue
        rows.append(key)
    return rows


@pytest.mark.parametrize("dtype", [0, 1, 2])
def test_time_model_is_positive_and_monotone(dtype):
    """Over the planner's domain (1 to ~4800 workgroups, K from 16 to 2^20)
    every row's predicted time is positive, never falls when workgroups are
    added (more rows of C) or K grows, and a K split into P parts is never
    predicted faster than one of its parts alone (P times the workgroups on
    K / P against the workgroups on K / P)."""
    rows = _perf_rows(dtype)
    assert len(rows) >= 5
    Ks = [16, 256, 1000, 1024, 2048, 4096, 6000, 16384, 65536, 1 << 20]
    for bm, bn, w, st in rows:
        for n_tiles_n in (1, 3, 8, 16, 48):
            N = n_tiles_n * bn
            prev_k = None
            for K in Ks:
                prev_m = 0.0
                for tiles_m in (1, 2, 4, 7, 8, 16, 24, 33, 48, 64, 96, 100):
                    t = tdg.tdg_predict_us(dtype, bm, bn, w, st, tiles_m * bm, N, K)
                    assert t > 0.0, (bm, bn, w, st, tiles_m, N, K, t)
                    assert t >= prev_m - 1e-9, (bm, bn, w, st, tiles_m, N, K, t, prev_m)
                    prev_m = t
                t = tdg.tdg_predict_us(dtype, bm, bn, w, st, 16 * bm, N, K)
                if prev_k is not None:
                    assert t >= prev_k - 1e-9, (bm, bn, w, st, N, K, t, prev_k)
                prev_k = t
            for P in (2, 4, 16, 64):
                K = 65536
                part = tdg.tdg_predict_us(dtype, bm, bn, w, st, 2 * bm, N, K // P)
                split = tdg.tdg_predict_us(dtype, bm, bn, w, st, 2 * bm * P, N, K // P)
                assert split >= part - 1e-9


def test_planner_respects_partial_requests():
    """A request that fixes part of the configuration is completed within it;
    one outside the measured table (a 64-byte K tile) falls back to the tile
    rule and still resolves."""
    F16 = tdg.TDG_DTYPE_F16F32
    assert _plan_str(F16, 4096, 4096, 4096, waves=4).startswith("256x256 w4")
    assert _plan_str(F16, 4096, 4096, 4096, bm=128, bn=128).startswith("128x128 w4")
    assert _plan_str(F16, 2048, 2048, 2048, bm=128, bn=128, lds_stages=2) == "128x128 w4 s2 direct_lds"
    cfg, _ = tdg.tdg_plan(F16, 4096, 4096, 4096, cfg={"bk": 32})
    assert cfg["bk"] == 32 and cfg["bm"] == 256


@no_device_only
def test_splitk_plan_and_workspace_validation():
    """Split K is planned only where tiles leave the chip idle, and its
    workspace is checked before any HIP call: missing, short, misaligned or
    overlapping A, B or C is TDG_ERR_INVALID_ARG (a good one reaches the
    device check, TDG_ERR_NO_DEVICE here)."""
    F16 = tdg.TDG_DTYPE_F16F32
    parts, ws = tdg.tdg_splitk_plan(F16, 256, 256, 65536)
    assert parts > 1 and ws == parts * 256 * 256 * 4
    assert tdg.tdg_splitk_plan(F16, 4096, 4096, 4096) == (1, 0)
    assert tdg.tdg_splitk_plan(F16, 256, 256, 0) == (1, 0)
    lib = tdg.load_library()
    M, N, K, P = 256, 256, 8192, 4
    A, B, C, W = 1 << 40, 2 << 40, 3 << 40, 4 << 40
    need = P * M * N * 4
    call = lambda ws, nbytes, parts=P: lib.gemm_f16f32_splitk(M, N, K, A, K, B, N, C, N, parts, ws,
                                                              nbytes, None)
    assert call(W, need) == tdg.TDG_ERR_NO_DEVICE
    assert call(None, need) == tdg.TDG_ERR_INVALID_ARG
    assert call(W, need - 1) == tdg.TDG_ERR_INVALID_ARG
    assert call(W + 4, need) == tdg.TDG_ERR_INVALID_ARG
    assert call(C + 64, need) == tdg.TDG_ERR_INVALID_ARG      # overlaps C
    assert call(A, need) == tdg.TDG_ERR_INVALID_ARG           # overlaps A
    assert call(W, need, parts=-1) == tdg.TDG_ERR_INVALID_ARG
    assert call(None, 0, parts=1) == tdg.TDG_ERR_NO_DEVICE    # one part needs no workspace


@no_device_only
def test_split_k_workspace_size_does_not_wrap():
    """A caller's part count times M * N * 4 can exceed 64 bits for outputs
    that fit in device memory (C of 131072^2 floats is 64 GB; 2^28 parts
    make the product exactly 2^64).  The size must not wrap to a small
    number that a short workspace or the built-in scratch array passes:
    both entry points refuse the call before any HIP call."""
    lib = tdg.load_library()
    M = N = 1 << 17
    K = 1024
    A, B, C, W = 1 << 40, 1 << 41, 1 << 42, 1 << 45
    for parts in (1 << 28, (1 << 28) + 1, (1 << 31) - 1):
        for claimed in (16, (1 << 64) - 1):     # no workspace holds 2^64 bytes, whatever is claimed
            assert lib.gemm_f16f32_splitk(M, N, K, A, K, B, N, C, N, parts, W, claimed, None) == \
                tdg.TDG_ERR_INVALID_ARG, (parts, claimed)
        assert lib.gemm_splitk_noalloc(tdg.TDG_DTYPE_F16F32, M, N, K, A, K, B, N, C, N, parts, None) == \
            tdg.TDG_ERR_SCRATCH, parts
    # a workspace of the exact size is accepted (the call gets to the device check)
    assert lib.gemm_f16f32_splitk(256, 256, 8192, A, 8192, B, 256, C, 256, 4, W, 4 * 256 * 256 * 4,
                                  None) == tdg.TDG_ERR_NO_DEVICE


@no_device_only
def test_split_k_with_an_empty_k_plans_nothing():
    """K = 0 is a valid product (C is zero-filled).  Asked to choose the part
    count (parts = 0), both split-K entry points must not plan a split of
    zero K tiles (that divided by zero in the host process): the call goes
    on to the plain zero fill and reaches the device check here."""
    lib = tdg.load_library()
    A, B, C, W = 1 << 40, 1 << 41, 1 << 42, 1 << 45
    for M, N in ((64, 1), (256, 256), (1, 4096)):
        for fn in (lib.gemm_f16f32_splitk, lib.gemm_i8i32_splitk, lib.gemm_f32f32_splitk):
            assert fn(M, N, 0, None, 1, None, N, C, N, 0, None, 0, None) == tdg.TDG_ERR_NO_DEVICE
            assert fn(M, N, 0, A, 1, B, N, C, N, 0, W, 16, None) == tdg.TDG_ERR_NO_DEVICE
        for dt in (0, 1, 2):
            assert lib.gemm_splitk_noalloc(dt, M, N, 0, None, 1, None, N, C, N, 0, None) == \
                tdg.TDG_ERR_NO_DEVICE
    assert tdg.tdg_splitk_plan(tdg.TDG_DTYPE_F16F32, 256, 256, 0) == (1, 0)


def test_sizes_keep_a_margin_below_2_31():
    """The kernels form tile start + tile extent in 32 bits, so M, N and K
    stop 2^16 short of 2^31: planning M at the limit works (a dense N or K
    that large already breaks the leading-dimension limit), one past it is an
    argument error for the planners and every entry point."""
    lim = (1 << 31) - (1 << 16)
    tdg.tdg_plan(tdg.TDG_DTYPE_F16F32, lim, 64, 64)
    tdg.tdg_plan(tdg.TDG_DTYPE_I8I32, lim, 64, 4096)
    for args in ((lim + 1, 64, 64), (64, lim + 1, 64), (64, 64, lim + 1)):
        with pytest.raises(tdg.TdgError):
            tdg.tdg_plan(tdg.TDG_DTYPE_F16F32, *args)
        with pytest.raises(tdg.TdgError):
            tdg.tdg_splitk_plan(tdg.TDG_DTYPE_I8I32, *args)


def test_config_resources_validation():
    """tdg_config_resources: bad dtype, index or output are argument errors
    before any HIP call; a valid query needs the gfx950 device."""
    lib = tdg.load_library()
    r = tdg.TdgKernelResources()
    n = tdg.tdg_config_count(tdg.TDG_DTYPE_F16F32)
    assert lib.tdg_config_resources(7, 0, ctypes.byref(r)) == tdg.TDG_ERR_INVALID_ARG
    assert lib.tdg_config_resources(tdg.TDG_DTYPE_F16F32, -1, ctypes.byref(r)) == tdg.TDG_ERR_INVALID_ARG
    assert lib.tdg_config_resources(tdg.TDG_DTYPE_F16F32, n, ctypes.byref(r)) == tdg.TDG_ERR_INVALID_ARG
    assert lib.tdg_config_resources(tdg.TDG_DTYPE_F16F32, 0, None) == tdg.TDG_ERR_INVALID_ARG
    assert lib.tdg_config_resources(tdg.TDG_DTYPE_F16F32, 0, ctypes.byref(r)) == tdg.TDG_ERR_NO_DEVICE


# --- which loop a call on given operands runs (tdg_plan_operands) ------------

ES = {tdg.TDG_DTYPE_F16F32: 2, tdg.TDG_DTYPE_I8I32: 1, tdg.TDG_DTYPE_F32F32: 4}
BASE = 1 << 40          # an address on a 4 KiB page boundary; never dereferenced


def _form(dtype, M, N, K, a, lda, b, ldb, **req):
    cfg, info = tdg.tdg_plan_operands(dtype, M, N, K, a, lda, b, ldb, tdg.TdgConfig(**req) if req else None)
    return cfg["variant"], info["guarded"]


def _last_chunk_leaves_page(base, rows, ld, cols, es):
    """Walk the last row's 16-byte chunks from its first byte, as the copy
    does, and say whether the one holding the operand's last byte reads a
    byte past it in another 4 KiB page (bytes before it are the operand's)."""
    row = base + (rows - 1) * ld * es
    last = row + cols * es - 1
    start = row
    while start + 16 <= last:          # the chunk [start, start + 16) ends before the last byte
        start += 16
    return any((x >> 12) != (last >> 12) for x in range(last + 1, start + 16))


@pytest.mark.parametrize("dtype", sorted(ES))
def test_plan_operands_whole_tiles_run_the_dma_at_any_alignment(dtype):
    """Whole tiles: the direct-to-LDS loop runs unchecked whatever the rows'
    alignment; the register and sequential loops run unchecked only with
    16-byte aligned rows."""
    es = ES[dtype]
    M = N = K = 1024
    aligned = (BASE, K, BASE + (1 << 30), N)
    for a_off, lda in ((es, K + 1), (0, K + 1), (es, K)):
        odd = (BASE + a_off, lda, BASE + (1 << 30) + es, N + 3)
        assert _form(dtype, M, N, K, *aligned) == (tdg.TDG_VARIANT_DIRECT_LDS, 0)
        assert _form(dtype, M, N, K, *odd) == (tdg.TDG_VARIANT_DIRECT_LDS, 0)
        for v in (tdg.TDG_VARIANT_REG_PREFETCH, tdg.TDG_VARIANT_SINGLE):
            stages = 2 if v == tdg.TDG_VARIANT_REG_PREFETCH else 1
            assert _form(dtype, M, N, K, *aligned, variant=v, lds_stages=stages) == (v, 0)
            assert _form(dtype, M, N, K, *odd, variant=v, lds_stages=stages) == (v, 1)
    # the dense, aligned case is what tdg_plan assumes
    cfg, info = tdg.tdg_plan(dtype, M, N, K)
    cfg2, info2 = tdg.tdg_plan_operands(dtype, M, N, K, *aligned)
    assert cfg == cfg2 and info == info2


@pytest.mark.parametrize("dtype", sorted(ES))
def test_plan_operands_last_chunk_page_rule(dtype):
    """Ragged shapes with rows off the 16-byte grid: the bounds-checked
    direct-to-LDS loop, unless the chunk holding an operand's last byte
    reaches into another page, when the register-prefetch loop runs.  Every
    placement of A, then of B, within a page, against a walk of the chunks."""
    es = ES[dtype]
    M, N, K = 300, 270, 137                      # K and N end inside a chunk
    lda, ldb = K + 1, N + 1
    b_far, a_far = BASE + (1 << 32), BASE + (1 << 33)
    seen = set()
    for s in range(0, 4096, es):
        a = BASE + s
        want = tdg.TDG_VARIANT_REG_PREFETCH if _last_chunk_leaves_page(a, M, lda, K, es) \
            else tdg.TDG_VARIANT_DIRECT_LDS
        b_ok = not _last_chunk_leaves_page(b_far, K, ldb, N, es)
        assert b_ok
        assert _form(dtype, M, N, K, a, lda, b_far, ldb) == (want, 1), s
        seen.add(want)
        b = BASE + s
        want = tdg.TDG_VARIANT_REG_PREFETCH if _last_chunk_leaves_page(b, K, ldb, N, es) \
            else tdg.TDG_VARIANT_DIRECT_LDS
        assert not _last_chunk_leaves_page(a_far, M, lda, K, es)
        assert _form(dtype, M, N, K, a_far, lda, b, ldb) == (want, 1), s
        seen.add(want)
    assert seen == {tdg.TDG_VARIANT_REG_PREFETCH, tdg.TDG_VARIANT_DIRECT_LDS}


@pytest.mark.parametrize("dtype", sorted(ES))
def test_plan_operands_aligned_rows_always_keep_the_dma(dtype):
    """With 16-byte aligned rows no chunk leaves its page: every ragged shape
    (K > 0, at least two K tiles) runs the direct-to-LDS loop, wherever on a
    page the operands sit."""
    import random
    es = ES[dtype]
    rng = random.Random(7 + dtype)
    epc = 16 // es
    for _ in range(300):
        M, N, K = rng.randint(1, 900), rng.randint(1, 900), rng.randint(300, 900)
        lda = -(-K // epc) * epc + epc * rng.randint(0, 3)
        ldb = -(-N // epc) * epc + epc * rng.randint(0, 3)
        a = BASE + 16 * rng.randint(0, 255)
        b = BASE + (1 << 32) + 16 * rng.randint(0, 255)
        assert _form(dtype, M, N, K, a, lda, b, ldb)[0] == tdg.TDG_VARIANT_DIRECT_LDS, (M, N, K)


def test_plan_operands_rejects_bad_arguments():
    f16 = tdg.TDG_DTYPE_F16F32
    for args in ((f16, 64, 64, 64, BASE, 63, BASE, 64),       # lda < K
                 (f16, 64, 64, 64, BASE, 64, BASE, 63),       # ldb < N
                 (f16, 64, 64, 64, 0, 64, BASE, 64),          # NULL A
                 (f16, 64, 64, 64, BASE, 64, 0, 64),          # NULL B
                 (f16, -1, 64, 64, BASE, 64, BASE, 64),
                 (9, 64, 64, 64, BASE, 64, BASE, 64)):
        with pytest.raises(tdg.TdgError) as e:
            tdg.tdg_plan_operands(*args)
        assert e.value.status == tdg.TDG_ERR_INVALID_ARG
    # empty operands may be NULL
    tdg.tdg_plan_operands(f16, 0, 64, 64, 0, 64, BASE, 64)


def test_plan_operands_misaligned_rows_prefer_tiles_that_copy_less():
    """Rows off the 16-byte grid make every copied byte dearer, so the
    planner moves to configurations that copy fewer bytes per compute unit
    (picks measured faster on MI355X: 27-30% at 7001 x 7001 x 1001, 11% for
    INT8 5000 x 777 x 3001); with aligned rows the same shapes keep their
    picks."""
    f16, i8 = tdg.TDG_DTYPE_F16F32, tdg.TDG_DTYPE_I8I32
    for code, (M, N, K), aligned, misaligned in [
            (f16, (7001, 7001, 1001), (128, 128), (256, 256)),
            (i8, (7001, 7001, 1001), (128, 128), (256, 256)),
            (i8, (5000, 777, 3001), (128, 128), (256, 128))]:
        epc = 16 // ES[code]
        a, _ = tdg.tdg_plan_operands(code, M, N, K, BASE, -(-K // epc) * epc, BASE + (1 << 32), -(-N // epc) * epc)
        m, _ = tdg.tdg_plan_operands(code, M, N, K, BASE, K, BASE + (1 << 32), N)
        assert (a["bm"], a["bn"]) == aligned, (M, N, K, a)
        assert (m["bm"], m["bn"]) == misaligned, (M, N, K, m)
