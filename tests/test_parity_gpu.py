"""GPU parity: the HIP kernels (through the C ABI) against the CPU oracle.

INT8 -> INT32 must match bit for bit; FP16 -> FP32 must satisfy
|C_gpu - C| <= 1e-4 * sum_k |a_ik b_kj| per element, and integer-valued FP16
inputs (every partial sum exact in FP32) must match exactly.  Pipelining only
reorders loads ("Pipeline GPU Kernel", Step 5), so every variant of one tile
configuration must produce bitwise-identical output.
"""
import numpy as np
import pytest

import oracle
import synthetic_inputs as si
from gpu_util import (F16, F32, I8, check_f16, check_f32, check_i8, check_sampled, gemm,
                      sample_indices, to_device)

pytestmark = pytest.mark.gpu

CODE = {F16: 0, I8: 1, F32: 2}   # tdg_dtype of each test dtype


@pytest.fixture(scope="module")
def lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import tiled_dense_gemm_loop_amd as t
    t.load_library()
    return t


def _operands(dtype, M, N, K, seed, dist="normal"):
    if dtype == I8:
        return si.i8_uniform(M, K, seed), si.i8_uniform(K, N, seed + 1)
    if dtype == F32:
        if dist == "int":
            return si.f32_integers(M, K, seed), si.f32_integers(K, N, seed + 1)
        return si.f32_normal(M, K, seed), si.f32_normal(K, N, seed + 1)
    if dist == "int":
        return si.f16_integers(M, K, seed), si.f16_integers(K, N, seed + 1)
    return si.f16_normal(M, K, seed), si.f16_normal(K, N, seed + 1)


def _check(dtype, C, A, B, exact=False, pages_rule=False):
    if dtype == I8:
        check_i8(C, A, B)
    elif dtype == F32:
        check_f32(C, A, B, exact=exact, pages_rule=pages_rule)
    else:
        check_f16(C, A, B, exact=exact, pages_rule=pages_rule)


def _variants(lib, dtype, tile):
    """Every built loop form (variant x LDS stages) at one tile shape:
    [(name, cfg)], the sequential baseline first."""
    import tiled_dense_gemm_loop_amd as t
    code = CODE[dtype]
    out = []
    for i in range(t.tdg_config_count(code)):
        c = t.tdg_config_at(code, i)
        if (c["bm"], c["bn"], c["bk"], c["waves"]) != (tile["bm"], tile["bn"], tile["bk"],
                                                        tile["waves"]):
            continue
        out.append(("%s_s%d" % (t.VARIANT_NAMES[c["variant"]], c["lds_stages"]), c))
    out.sort(key=lambda nc: (nc[1]["variant"], nc[1]["lds_stages"]))
    assert out and out[0][1]["variant"] == t.TDG_VARIANT_SINGLE
    return out


def _tiles(dtype_code):
    import tiled_dense_gemm_loop_amd as t
    seen, out = set(), []
    for i in range(t.tdg_config_count(dtype_code)):
        c = t.tdg_config_at(dtype_code, i)
        key = (c["bm"], c["bn"], c["bk"], c["waves"])
        if key not in seen:
            seen.add(key)
            out.append(dict(zip(("bm", "bn", "bk", "waves"), key)))
    return out


def _all_tiles():
    try:
        return [(d, c) for d in (F16, I8, F32) for c in _tiles(CODE[d])]
    except ImportError:
        return []


# --- the small workloads, whole-matrix parity ---------------------------------------

def test_int8_256_every_entry_point(lib):
    wl = si.WORKLOADS["int8_256"]
    A, B = wl.operands()
    dA, dB = to_device(A), to_device(B)
    outs = []
    for kind in ("single", "pipelined"):
        C = gemm(lib, I8, kind, dA, dB)
        check_i8(C, A, B)
        outs.append(C)
    tile, _ = lib.tdg_plan(lib.TDG_DTYPE_I8I32, wl.M, wl.N, wl.K)
    for name, cfg in _variants(lib, I8, tile):
        C = gemm(lib, I8, "ex", dA, dB, cfg=cfg)
        check_i8(C, A, B)


def test_fp16_1024_single_vs_pipelined(lib):
    import torch
    wl = si.WORKLOADS["fp16_1024"]
    A, B = wl.operands()
    dA, dB = to_device(A), to_device(B)
    C1 = gemm(lib, F16, "single", dA, dB)
    C2 = gemm(lib, F16, "pipelined", dA, dB)
    check_f16(C1, A, B)
    check_f16(C2, A, B)
    assert torch.equal(C1, C2), "single and pipelined differ at the same tile"


# --- every built tile shape x every loop form ------------------------------------------

@pytest.mark.parametrize("dtype,tile", _all_tiles(),
                         ids=lambda v: v if isinstance(v, str) else
                         "%dx%dx%d_w%d" % (v["bm"], v["bn"], v["bk"], v["waves"]))
def test_tile_shape_all_variants(lib, dtype, tile):
    import torch
    M, N, K = 2 * tile["bm"], 2 * tile["bn"], 3 * tile["bk"]
    A, B = _operands(dtype, M, N, K, seed=M + N + K)
    dA, dB = to_device(A), to_device(B)
    ref_out = None
    for name, cfg in _variants(lib, dtype, tile):
        C = gemm(lib, dtype, "ex", dA, dB, cfg=cfg)
        _check(dtype, C, A, B)
        if ref_out is None:
            ref_out = C
        else:
            assert torch.equal(ref_out, C), "variant %s differs from single" % name


@pytest.mark.parametrize("dtype,tile", _all_tiles(),
                         ids=lambda v: v if isinstance(v, str) else
                         "%dx%dx%d_w%d" % (v["bm"], v["bn"], v["bk"], v["waves"]))
def test_poisoned_lds_race_screen(lib, dtype, tile):
    """Every loop form with the LDS ring filled with 0xFF bytes before the
    first tile lands: a read of a buffer the pipeline has not filled yet
    would see NaN (FP16, FP32) or -1 (INT8).  Whole tiles, a chunk-aligned
    ragged shape (bounds-checked direct-to-LDS) and a chunk-splitting one
    (bounds-checked register loads); each against the oracle and bitwise
    against the same launch without the poison."""
    import torch
    epc = 16 // {F16: 2, I8: 1, F32: 4}[dtype]
    bm, bn, bk = tile["bm"], tile["bn"], tile["bk"]
    shapes = [(2 * bm, 2 * bn, 3 * bk), (2 * bm - 3, 2 * bn - epc, 3 * bk - epc),
              (2 * bm - 5, 2 * bn - 3, 3 * bk - 1)]
    for si_, (M, N, K) in enumerate(shapes):
        A, B = _operands(dtype, M, N, K, seed=7 * M + N + K + si_)
        dA, dB = to_device(A), to_device(B)
        for name, cfg in _variants(lib, dtype, tile):
            clean = gemm(lib, dtype, "ex", dA, dB, cfg=cfg)
            prev = lib.tdg_set_debug_flags(lib.TDG_DEBUG_POISON_LDS)
            try:
                C = gemm(lib, dtype, "ex", dA, dB, cfg=cfg)
            finally:
                lib.tdg_set_debug_flags(prev)
            _check(dtype, C, A, B)
            assert torch.equal(C, clean), "%s at %s changes under poisoned LDS" % (name, (M, N, K))


# --- ragged, tiny and degenerate shapes (bounds-checked path) ---------------------------

RAGGED = [(1, 1, 1), (5, 7, 3), (64, 64, 1), (33, 65, 17), (300, 290, 333), (257, 129, 65),
          (130, 260, 200), (1000, 3, 70), (3, 1000, 129), (64, 64, 63)]


@pytest.mark.parametrize("dtype", [F16, I8, F32])
@pytest.mark.parametrize("M,N,K", RAGGED)
def test_ragged_shapes(lib, dtype, M, N, K):
    A, B = _operands(dtype, M, N, K, seed=7 * M + N + K)
    dA, dB = to_device(A), to_device(B)
    for kind in ("single", "pipelined"):
        _check(dtype, gemm(lib, dtype, kind, dA, dB), A, B)


@pytest.mark.parametrize("dtype", [F16, I8, F32])
def test_ragged_every_tile(lib, dtype):
    M, N, K = 301, 283, 259
    A, B = _operands(dtype, M, N, K, seed=99)
    dA, dB = to_device(A), to_device(B)
    for tile in _tiles(CODE[dtype]):
        for name, cfg in _variants(lib, dtype, tile):
            _check(dtype, gemm(lib, dtype, "ex", dA, dB, cfg=cfg), A, B)


# --- ragged shapes on the bounds-checked direct-to-LDS path --------------------------
# N and K whole 16-byte chunks (8 FP16 / 16 INT8 elements), aligned rows: chunks
# outside A or B come from a zero block, so the result must equal the one of the
# element-wise guarded loop at the same tile bit for bit.

RAGGED_DMA = [(1, 16, 16), (5, 32, 48), (300, 272, 144), (257, 144, 272), (130, 400, 528),
              (1000, 16, 1040), (64, 64, 16)]


@pytest.mark.parametrize("dtype", [F16, I8, F32])
@pytest.mark.parametrize("M,N,K", RAGGED_DMA)
def test_ragged_direct_shapes(lib, dtype, M, N, K):
    import torch
    A, B = _operands(dtype, M, N, K, seed=3 * M + N + K)
    dA, dB = to_device(A), to_device(B)
    code = CODE[dtype]
    cfg, info = lib.tdg_plan(code, M, N, K)
    # one K tile: the planner runs the sequential form (nothing to overlap)
    want = lib.TDG_VARIANT_DIRECT_LDS if info["num_tiles"] >= 2 else lib.TDG_VARIANT_SINGLE
    assert info["guarded"] == 1 and cfg["variant"] == want
    C = gemm(lib, dtype, "pipelined", dA, dB)
    _check(dtype, C, A, B)
    direct = dict(cfg, variant=lib.TDG_VARIANT_DIRECT_LDS, lds_stages=2)
    reg = dict(cfg, variant=lib.TDG_VARIANT_REG_PREFETCH, lds_stages=2)
    assert torch.equal(C, gemm(lib, dtype, "ex", dA, dB, cfg=direct))
    assert torch.equal(C, gemm(lib, dtype, "ex", dA, dB, cfg=reg))


@pytest.mark.parametrize("dtype", [F16, I8, F32])
def test_ragged_direct_every_tile(lib, dtype):
    """Every tile and every ring depth asked for on a ragged, chunk-aligned
    shape: all forms agree bit for bit and with the oracle."""
    import torch
    M, N, K = 301, 288, 272
    A, B = _operands(dtype, M, N, K, seed=98)
    dA, dB = to_device(A), to_device(B)
    for tile in _tiles(CODE[dtype]):
        ref_out = None
        for name, cfg in _variants(lib, dtype, tile):
            C = gemm(lib, dtype, "ex", dA, dB, cfg=cfg)
            if ref_out is None:
                _check(dtype, C, A, B)
                ref_out = C
            else:
                assert torch.equal(ref_out, C), "%s differs at tile %s" % (name, tile)


@pytest.mark.parametrize("dtype", [F16, I8, F32])
def test_ragged_direct_long_k_every_ring(lib, dtype):
    """A ragged, chunk-aligned shape with a partial last K tile and enough
    K tiles that every ring depth runs interior workgroups on the plain DMA
    first and switches to the bounds-checked DMA for the tail: every tile
    and ring agree with the element-wise guarded loop bit for bit, and with
    the oracle."""
    import torch
    M, N, K = 300, 272, 2000 if dtype != I8 else 4016
    A, B = _operands(dtype, M, N, K, seed=97)
    dA, dB = to_device(A), to_device(B)
    for tile in _tiles(CODE[dtype]):
        ref_out = None
        for name, cfg in _variants(lib, dtype, tile):
            C = gemm(lib, dtype, "ex", dA, dB, cfg=cfg)
            if ref_out is None:
                _check(dtype, C, A, B)
                ref_out = C
            else:
                assert torch.equal(ref_out, C), "%s differs at tile %s" % (name, tile)


@pytest.mark.parametrize("dtype", [F16, I8, F32])
def test_ragged_direct_padded_rows(lib, dtype):
    """Leading dimensions wider than the matrix (still 16-byte multiples)
    on the ragged direct path: nothing past a row's K or N is used."""
    M, N, K = 200, 144, 176
    bigA, bigB = _operands(dtype, M + 2, N + 48, K + 32, seed=17)
    A, B = bigA[1:1 + M, :K], bigB[1:1 + K, 16:16 + N]
    dA = to_device(bigA)[1:1 + M, :K]
    dB = to_device(bigB)[1:1 + K, 16:16 + N]
    C = gemm(lib, dtype, "pipelined", dA, dB)
    _check(dtype, C, A, B)


# --- K or N that splits a 16-byte chunk, rows still 16-byte aligned --------------------
# These keep the direct-to-LDS copy: chunks are fetched whole, and the kernel
# clears A's bytes at k >= K in the one chunk per row that K splits.  The
# operands are views into wider storage whose padding holds NaN (INT8: 127),
# so a byte past K or N that reached a stored sum would show.

POISON = {F16: np.uint16(0x7E00), I8: np.int8(127), F32: np.float32("nan")}


def _split_chunk_operands(dtype, M, N, K, seed, pad_chunks=1):
    """(A, B, dA, dB): host operands and device views of them whose rows are
    16-byte aligned, ld = K (or N) rounded up to whole 16-byte chunks plus
    pad_chunks more, padding filled with POISON."""
    es = {F16: 2, I8: 1, F32: 4}[dtype]
    epc = 16 // es
    lda = -(-K // epc) * epc + pad_chunks * epc
    ldb = -(-N // epc) * epc + pad_chunks * epc
    A, B = _operands(dtype, M, N, K, seed=seed)
    bigA = np.full((M, lda), POISON[dtype], dtype=A.dtype)
    bigB = np.full((K, ldb), POISON[dtype], dtype=B.dtype)
    bigA[:, :K] = A
    bigB[:, :N] = B
    return A, B, to_device(bigA)[:, :K], to_device(bigB)[:, :N]


SPLIT_CHUNK = [(300, 270, 137), (257, 129, 263), (64, 63, 65), (5, 7, 3), (1000, 61, 1001),
               (130, 400, 529), (256, 256, 255), (64, 64, 129)]


@pytest.mark.parametrize("dtype", [F16, I8, F32])
@pytest.mark.parametrize("M,N,K", SPLIT_CHUNK)
def test_split_chunk_direct_shapes(lib, dtype, M, N, K):
    """K and / or N ending inside a 16-byte chunk, aligned rows: the planner
    keeps the bounds-checked direct-to-LDS loop; the result matches the
    oracle and, bit for bit, the guarded register-prefetch loop (which
    zeroes the same bytes in registers) and the two-buffer DMA ring."""
    import torch
    A, B, dA, dB = _split_chunk_operands(dtype, M, N, K, seed=5 * M + 3 * N + K)
    code = CODE[dtype]
    cfg, info = lib.tdg_plan(code, M, N, K)
    C = gemm(lib, dtype, "pipelined", dA, dB)
    _check(dtype, C, A, B)
    direct = dict(cfg, variant=lib.TDG_VARIANT_DIRECT_LDS, lds_stages=2)
    reg = dict(cfg, variant=lib.TDG_VARIANT_REG_PREFETCH, lds_stages=2)
    Cd = gemm(lib, dtype, "ex", dA, dB, cfg=direct)
    _check(dtype, Cd, A, B)
    assert torch.equal(Cd, gemm(lib, dtype, "ex", dA, dB, cfg=reg))
    if info["num_tiles"] >= 2:
        assert torch.equal(C, Cd)


@pytest.mark.parametrize("dtype", [F16, I8, F32])
def test_split_chunk_direct_every_tile_and_ring(lib, dtype):
    """A long K that ends inside a chunk, N too: every tile and every ring
    depth built (interior workgroups run the plain DMA, then the checked one
    from the partial tile on) against the oracle and bit for bit against the
    tile's sequential loop; once more under the LDS poisoning race screen."""
    import torch
    M, N, K = 300, 270, {F16: 2001, I8: 4013, F32: 1001}[dtype]
    A, B, dA, dB = _split_chunk_operands(dtype, M, N, K, seed=96)
    for tile in _tiles(CODE[dtype]):
        ref_out = None
        for name, cfg in _variants(lib, dtype, tile):
            C = gemm(lib, dtype, "ex", dA, dB, cfg=cfg)
            if ref_out is None:
                _check(dtype, C, A, B)
                ref_out = C
            else:
                assert torch.equal(ref_out, C), "%s differs at tile %s" % (name, tile)
            if cfg["variant"] == lib.TDG_VARIANT_DIRECT_LDS:
                prev = lib.tdg_set_debug_flags(lib.TDG_DEBUG_POISON_LDS)
                try:
                    C2 = gemm(lib, dtype, "ex", dA, dB, cfg=cfg)
                finally:
                    lib.tdg_set_debug_flags(prev)
                assert torch.equal(ref_out, C2), "%s differs under the LDS poison" % name


# --- rows off the 16-byte grid: the direct-to-LDS loop -----------------------

def _misaligned_operands(dtype, M, N, K, seed, shift=1):
    """Operands whose rows start off the 16-byte grid: leading dimensions of
    K + 1 and N + 1 elements, bases `shift` elements into their buffers,
    everything around them POISON."""
    A, B = _operands(dtype, M, N, K, seed)
    lda, ldb = K + 1, N + 1
    bigA = np.full(M * lda + shift + 16, POISON[dtype], dtype=A.dtype)
    bigB = np.full(K * ldb + shift + 16, POISON[dtype], dtype=B.dtype)
    bigA[shift:shift + M * lda].reshape(M, lda)[:, :K] = A
    bigB[shift:shift + K * ldb].reshape(K, ldb)[:, :N] = B
    dA = to_device(bigA)[shift:shift + M * lda].view(M, lda)[:, :K]
    dB = to_device(bigB)[shift:shift + K * ldb].view(K, ldb)[:, :N]
    return A, B, dA, dB


def _dma_placement(lib, dtype, M, N, K, seed):
    """Misaligned operands that the pipelined call runs in the direct-to-LDS
    loop (a base shift for which neither operand's last chunk leaves its
    page: all but about 1 in 250 placements)."""
    code = CODE[dtype]
    for shift in (1, 2, 3, 5):
        A, B, dA, dB = _misaligned_operands(dtype, M, N, K, seed, shift)
        cfg, info = lib.tdg_plan_operands(code, M, N, K, dA.data_ptr(), dA.stride(0),
                                          dB.data_ptr(), dB.stride(0))
        if cfg["variant"] == lib.TDG_VARIANT_DIRECT_LDS:
            assert dA.data_ptr() % 16 or dA.stride(0) * dA.element_size() % 16
            return A, B, dA, dB, cfg, info
    raise AssertionError("no placement keeps the copy in the DMA")


MISALIGNED = [(512, 512, 512), (256, 512, 1024), (300, 270, 137), (257, 129, 263), (1000, 61, 1001),
              (64, 64, 129)]


@pytest.mark.parametrize("dtype", [F16, I8, F32])
@pytest.mark.parametrize("M,N,K", MISALIGNED)
def test_misaligned_rows_run_the_dma(lib, dtype, M, N, K):
    """Rows off the 16-byte grid (odd leading dimensions, bases off a chunk):
    the pipelined call runs the direct-to-LDS loop -- unchecked on whole
    tiles, bounds-checked on ragged shapes -- whose DMA reads each chunk
    from its own byte address.  Against the oracle, and bit for bit against
    the bounds-checked register-prefetch loop at the same tile."""
    import torch
    A, B, dA, dB, cfg, info = _dma_placement(lib, dtype, M, N, K, seed=M + N + K)
    whole = M % cfg["bm"] == 0 and N % cfg["bn"] == 0 and K % cfg["bk"] == 0
    assert info["guarded"] == (0 if whole else 1)
    C = gemm(lib, dtype, "pipelined", dA, dB)
    _check(dtype, C, A, B)
    reg = dict(cfg, variant=lib.TDG_VARIANT_REG_PREFETCH, lds_stages=2)
    assert torch.equal(C, gemm(lib, dtype, "ex", dA, dB, cfg=reg))


@pytest.mark.parametrize("dtype", [F16, I8, F32])
def test_misaligned_rows_every_tile_and_ring(lib, dtype):
    """Misaligned rows, a long K and an N that end inside a chunk: every
    tile and every ring depth built against the oracle and bit for bit
    against the tile's sequential loop; the direct-to-LDS forms once more
    under the LDS poisoning race screen."""
    import torch
    M, N, K = 300, 270, {F16: 2001, I8: 4013, F32: 1001}[dtype]
    A, B, dA, dB, _, _ = _dma_placement(lib, dtype, M, N, K, seed=98)
    for tile in _tiles(CODE[dtype]):
        ref_out = None
        for name, cfg in _variants(lib, dtype, tile):
            C = gemm(lib, dtype, "ex", dA, dB, cfg=cfg)
            if ref_out is None:
                _check(dtype, C, A, B)
                ref_out = C
            else:
                assert torch.equal(ref_out, C), "%s differs at tile %s" % (name, tile)
            if cfg["variant"] == lib.TDG_VARIANT_DIRECT_LDS:
                prev = lib.tdg_set_debug_flags(lib.TDG_DEBUG_POISON_LDS)
                try:
                    C2 = gemm(lib, dtype, "ex", dA, dB, cfg=cfg)
                finally:
                    lib.tdg_set_debug_flags(prev)
                assert torch.equal(ref_out, C2), "%s differs under the LDS poison" % name


@pytest.mark.parametrize("dtype", [F16, I8, F32])
@pytest.mark.parametrize("which", ["A", "B"])
def test_last_chunk_across_a_page(lib, dtype, which):
    """An operand placed so that the 16-byte chunk holding its last byte
    reaches into the next 4 KiB page: the call runs the bounds-checked
    register-prefetch loop (tdg_plan_operands says so), whose loads stay in
    the page of their first byte; placed so that it does not, the
    direct-to-LDS loop.  Both against the oracle.  The operand sits inside a
    larger buffer, so every page here is mapped whatever the planner
    decides; the other operand has aligned rows."""
    import torch
    code = CODE[dtype]
    es = {F16: 2, I8: 1, F32: 4}[dtype]
    epc = 16 // es
    M, N, K = 300, 270, 137
    A, B = _operands(dtype, M, N, K, seed=99)
    if which == "A":
        rows, ld, cols, src, other_np, o_cols = M, K + 1, K, A, B, N
    else:
        rows, ld, cols, src, other_np, o_cols = K, N + 1, N, B, A, K
    o_ld = -(-o_cols // epc) * epc             # aligned rows for the other operand
    o_host = np.full((other_np.shape[0], o_ld), POISON[dtype], dtype=other_np.dtype)
    o_host[:, :o_cols] = other_np
    other = to_device(o_host)[:, :o_cols]
    span = rows * ld
    big = np.full(span + 2 * 4096 // es, POISON[dtype], dtype=src.dtype)
    d_big = to_device(big)

    def operands(s):
        view = d_big[s:s + span].view(rows, ld)[:, :cols]
        return (view, other) if which == "A" else (other, view)

    found = {}
    for s in range(4096 // es):
        a, b = operands(s)
        cfg, _ = lib.tdg_plan_operands(code, M, N, K, a.data_ptr(), a.stride(0), b.data_ptr(), b.stride(0))
        found.setdefault(cfg["variant"], s)
    assert set(found) == {lib.TDG_VARIANT_REG_PREFETCH, lib.TDG_VARIANT_DIRECT_LDS}, found
    for want, s in sorted(found.items()):
        host = big.copy()
        host[s:s + span].reshape(rows, ld)[:, :cols] = src
        d_big.copy_(to_device(host))           # same buffer, same addresses
        a, b = operands(s)
        cfg, _ = lib.tdg_plan_operands(code, M, N, K, a.data_ptr(), a.stride(0), b.data_ptr(), b.stride(0))
        assert cfg["variant"] == want, (s, cfg)
        _check(dtype, gemm(lib, dtype, "pipelined", a, b), A, B)
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", [F16, I8])
def test_split_chunk_direct_rotated_and_split_k(lib, dtype):
    """The straddling K tile at every position of a rotated K walk (a skinny
    product whose B fits in L2), and inside one part of a split-K product."""
    import torch
    M, N, K = 4000, 61, 2003
    A, B, dA, dB = _split_chunk_operands(dtype, M, N, K, seed=95)
    cfg, info = lib.tdg_plan(CODE[dtype], M, N, K)
    assert info["k_rotated"] == 1
    C = gemm(lib, dtype, "pipelined", dA, dB)
    _check(dtype, C, A, B)
    prev = lib.tdg_set_debug_flags(lib.TDG_DEBUG_NO_K_ROTATION)
    try:
        plain = gemm(lib, dtype, "pipelined", dA, dB)
    finally:
        lib.tdg_set_debug_flags(prev)
    _check(dtype, plain, A, B)
    if dtype == I8:
        assert torch.equal(C, plain)
    fn = {F16: lib.gemm_f16f32_splitk, I8: lib.gemm_i8i32_splitk}[dtype]
    A2, B2, dA2, dB2 = _split_chunk_operands(dtype, 256, 256, 6001, seed=94)
    C2 = fn(dA2, dB2, parts=5)
    _check(dtype, C2, A2, B2)


@pytest.mark.parametrize("dtype", [F16, I8, F32])
def test_k_zero_writes_zeros(lib, dtype):
    import torch
    M, N = 300, 260
    A = np.zeros((M, 0), dtype={F16: np.uint16, I8: np.int8, F32: np.float32}[dtype])
    B = np.zeros((0, N), dtype=A.dtype)
    out_t = torch.int32 if dtype == I8 else torch.float32
    for kind in ("single", "pipelined"):
        C = torch.full((M, N), 7, dtype=out_t, device="cuda")
        gemm(lib, dtype, kind, to_device(A), to_device(B), C)
        assert torch.count_nonzero(C).item() == 0


def test_empty_outputs_are_noops(lib):
    import torch
    for (M, N, K) in [(0, 5, 7), (5, 0, 7), (0, 0, 0)]:
        A = torch.zeros((M, K), dtype=torch.int8, device="cuda")
        B = torch.zeros((K, N), dtype=torch.int8, device="cuda")
        C = gemm(lib, I8, "pipelined", A, B)
        assert C.shape == (M, N)


@pytest.mark.parametrize("dtype", [F16, I8, F32])
def test_strided_and_misaligned_operands(lib, dtype):
    """Leading dimensions wider than the matrix, and base pointers that are
    not 16-byte aligned: the fast path must be skipped, results unchanged."""
    M, N, K = 512, 256, 320
    bigA, bigB = _operands(dtype, M + 3, N + 40, K + 40, seed=5)
    for (ao, bo) in [(0, 0), (1, 3)]:
        A = bigA[1:1 + M, ao:ao + K]
        B = bigB[2:2 + K, bo:bo + N]
        dBigA, dBigB = to_device(bigA), to_device(bigB)
        dA = dBigA[1:1 + M, ao:ao + K]
        dB = dBigB[2:2 + K, bo:bo + N]
        for kind in ("single", "pipelined"):
            _check(dtype, gemm(lib, dtype, kind, dA, dB), A, B)


@pytest.mark.parametrize("dtype", [F16, I8, F32])
def test_every_byte_alignment(lib, dtype):
    """Odd leading dimensions, so rows start at every element offset within
    a 16-byte chunk, and every base offset within a chunk; K and N split a
    chunk, so the tails end at every position.  In the register loops (the
    single-buffer call) whole chunks take the single unaligned load, partial
    ones the shifted pair of aligned loads; the pipelined call's DMA reads
    every chunk from its own byte address."""
    epc = 16 // {F16: 2, I8: 1, F32: 4}[dtype]
    M, N, K = 70, 46, 262                     # K, N even; both split a chunk
    bigA, bigB = _operands(dtype, M + 1, N + 2 * epc + 1, K + 2 * epc + 1, seed=17)
    dBigA, dBigB = to_device(bigA), to_device(bigB)
    assert bigA.shape[1] % 2 == 1 and bigB.shape[1] % 2 == 1
    import torch
    out_t = torch.int32 if dtype == I8 else torch.float32
    for off in range(epc):
        A = bigA[1:1 + M, off:off + K]
        B = bigB[1:1 + K, epc - 1 - off:epc - 1 - off + N]
        dA = dBigA[1:1 + M, off:off + K]
        dB = dBigB[1:1 + K, epc - 1 - off:epc - 1 - off + N]
        for kind in ("single", "pipelined"):
            # C at every 4-byte offset within 16 bytes too, with ldc = N + 5
            co = off % 4
            bigC = torch.full((M, N + 5), -3, dtype=out_t, device="cuda")
            C = bigC[:, co:co + N]
            _check(dtype, gemm(lib, dtype, kind, dA, dB, C), A, B)
            assert torch.all(bigC[:, :co] == -3) and torch.all(bigC[:, co + N:] == -3)


@pytest.mark.parametrize("dtype", [F16, I8, F32])
def test_tails_at_every_page_offset(lib, dtype):
    """Odd leading dimensions over enough rows put the partial K
    chunks of A and the partial N chunks of B at every element offset within
    a 4 KiB page, so some of them would run past their page: in the
    register loops those take the pair of aligned loads instead of the
    single unaligned one; the DMA reads them whole (past a row's end lies
    the next row)."""
    M, N, K = (4200, 46, 4202) if dtype == I8 else (2100, 46, 2102)   # rows cover every offset
    bigA, bigB = _operands(dtype, M, N + 17, K + 1, seed=23)      # lda = K+1, ldb = N+17: odd
    A, B = bigA[:, :K], bigB[:K, :N]
    dBigA, dBigB = to_device(bigA), to_device(bigB)
    dA, dB = dBigA[:, :K], dBigB[:K, :N]
    esize = dA.element_size()
    epc = 16 // esize
    assert K % epc and N % epc
    # page offsets of the first byte of each row's partial chunk
    offs_a = {(dA.data_ptr() + (r * (K + 1) + K // epc * epc) * esize) % 4096 for r in range(M)}
    offs_b = {(dB.data_ptr() + (r * (N + 17) + N // epc * epc) * esize) % 4096 for r in range(K)}
    assert max(offs_a) > 4096 - 16 and max(offs_b) > 4096 - 16
    for kind in ("single", "pipelined"):
        _check(dtype, gemm(lib, dtype, kind, dA, dB), A, B)


@pytest.mark.parametrize("dtype", [F16, I8, F32])
def test_random_shapes_strides_and_configs(lib, dtype):
    """A seeded sweep over the space the other tests sample by hand: random
    M, N, K (1..900, a third of them within 3 of a tile multiple), leading
    dimensions padded by 0..40 elements and base offsets of 0..15 elements
    for A, B and C (every byte offset of a 16-byte chunk for INT8, every
    element offset for FP16 and FP32).  Each case runs the planner's choice,
    the sequential loop, two random built configurations (tile, waves, loop
    form, stages) and split K, a third of the launches with the LDS poisoned
    between tiles.  Every result against the oracle, computed once per case;
    C's padding untouched."""
    import random
    import torch
    rng = random.Random({F16: 11, I8: 12, F32: 13}[dtype])
    code = CODE[dtype]
    configs = [lib.tdg_config_at(code, i) for i in range(lib.tdg_config_count(code))]
    out_t = torch.int32 if dtype == I8 else torch.float32
    split = {F16: lib.gemm_f16f32_splitk, I8: lib.gemm_i8i32_splitk, F32: lib.gemm_f32f32_splitk}[dtype]
    prev = lib.tdg_set_debug_flags(0)
    try:
        for case in range(40):
            if rng.random() < 0.3:
                M, N, K = (max(1, rng.choice((64, 128, 256, 512, 768)) + rng.randint(-3, 3))
                           for _ in range(3))
            else:
                M, N, K = rng.randint(1, 900), rng.randint(1, 900), rng.randint(1, 900)
            pa, pb, pc = rng.randint(0, 40), rng.randint(0, 40), rng.randint(0, 40)
            oa, ob, oc = rng.randint(0, 15), rng.randint(0, 15), rng.randint(0, 15)
            bigA, bigB = _operands(dtype, M, N + pb + ob, K + pa + oa, seed=1000 + case)
            bigB = bigB[:K, :]                   # K rows, ldb = N + pb + ob
            A, B = bigA[:, oa:oa + K], bigB[:, ob:ob + N]
            dBigA, dBigB = to_device(bigA), to_device(bigB)
            dA, dB = dBigA[:, oa:oa + K], dBigB[:, ob:ob + N]
            if dtype == I8:
                ref, S = oracle.gemm_i8(A, B), None
            else:
                ref, S = (oracle.gemm_f32 if dtype == F32 else oracle.gemm_f16)(A, B)
            runs = [("pipelined", None), ("single", None), ("ex", rng.choice(configs)),
                    ("ex", rng.choice(configs)), ("splitk", rng.choice((0, 2, 3, 5)))]
            for kind, arg in runs:
                poison = rng.random() < 0.3
                lib.tdg_set_debug_flags(lib.TDG_DEBUG_POISON_LDS if poison else 0)
                what = (case, M, N, K, pa, pb, pc, oa, ob, oc, kind, arg, poison)
                bigC = torch.full((M, N + pc + oc), -7, dtype=out_t, device="cuda")
                C = bigC[:, oc:oc + N]
                if kind == "splitk":
                    split(dA, dB, C, parts=arg)
                elif kind == "ex":
                    gemm(lib, dtype, "ex", dA, dB, C, cfg=arg)
                else:
                    gemm(lib, dtype, kind, dA, dB, C)
                got = C.cpu().numpy()
                if dtype == I8:
                    bad = np.argwhere(got.astype(np.int64) != ref)
                else:
                    bad = np.argwhere(np.abs(got.astype(np.float64) - ref) > 1e-4 * S)
                assert bad.size == 0, (what, len(bad), tuple(bad[0]))
                assert torch.all(bigC[:, :oc] == -7) and torch.all(bigC[:, oc + N:] == -7), what
    finally:
        lib.tdg_set_debug_flags(prev)


@pytest.mark.parametrize("dtype", [F16, I8, F32])
@pytest.mark.parametrize("M,N,K", [(1, 1, 100000), (1, 3000, 5000), (3000, 1, 5000), (2, 2, 65536)])
def test_extreme_aspect_ratios(lib, dtype, M, N, K):
    """A dot product, a single row, a single column and a 2 x 2 output over a
    long K: one workgroup or one tile row/column, long K walks."""
    A, B = _operands(dtype, M, N, K, seed=M + 2 * N + 3 * K)
    dA, dB = to_device(A), to_device(B)
    for kind in ("single", "pipelined"):
        _check(dtype, gemm(lib, dtype, kind, dA, dB), A, B)


@pytest.mark.parametrize("dtype,bm,bn,bk,waves", [(F16, 128, 128, 64, 4), (F16, 256, 256, 32, 8),
                                                  (I8, 128, 128, 128, 4), (I8, 256, 256, 64, 8)])
def test_largest_leading_dimensions(lib, dtype, bm, bn, bk, waves):
    """The largest 16-byte aligned leading dimensions a kernel's unsigned
    32-bit per-lane offsets reach ((R - 1) * ld * sizeof(T) + row bytes
    < 2^32, R = rows its threads cover with their first chunk: 128 for the
    8-wave 256 x 256 tiles with a 64-byte K tile), for A and B at once, on
    whole tiles of the unguarded path, two K tiles, in every loop form.  A
    and B are views into matrices of 8.7 to 18 GB."""
    import torch
    es = 2 if dtype == F16 else 1
    threads = waves * 64
    a_rows, b_rows = threads // (bk * es // 16), threads // (bn * es // 16)
    lim = (1 << 32) - 1
    lda = (lim - bk * es) // (a_rows - 1) // es
    ldb = (lim - bn * es) // (b_rows - 1) // es
    lda -= lda % (16 // es)                   # keep rows 16-byte aligned
    ldb -= ldb % (16 // es)
    assert (a_rows - 1) * lda * es + bk * es <= lim and (b_rows - 1) * ldb * es + bn * es <= lim
    M, N, K = bm, bn, 2 * bk
    A, B = _operands(dtype, M, N, K, seed=77)
    tdt = torch.float16 if dtype == F16 else torch.int8
    bigA = torch.empty((M, lda), dtype=tdt, device="cuda")
    bigB = torch.empty((K, ldb), dtype=tdt, device="cuda")
    try:
        bigA[:, :K] = to_device(A)
        bigB[:, :N] = to_device(B)
        outs = []
        for variant, stages in ((lib.TDG_VARIANT_SINGLE, 1), (lib.TDG_VARIANT_REG_PREFETCH, 2),
                                (lib.TDG_VARIANT_DIRECT_LDS, 2)):
            cfg = dict(bm=bm, bn=bn, bk=bk, waves=waves, lds_stages=stages, variant=variant)
            C = gemm(lib, dtype, "ex", bigA[:, :K], bigB[:, :N], cfg=cfg)
            _check(dtype, C, A, B)
            outs.append(C)
        assert all(torch.equal(outs[0], c) for c in outs[1:])
    finally:
        del bigA, bigB
        torch.cuda.empty_cache()


def test_output_leading_dimension(lib):
    import torch
    M, N, K = 256, 256, 192
    A, B = _operands(I8, M, N, K, seed=11)
    big = torch.full((M, N + 64), -5, dtype=torch.int32, device="cuda")
    C = big[:, 32:32 + N]
    gemm(lib, I8, "pipelined", to_device(A), to_device(B), C)
    check_i8(C, A, B)
    assert torch.all(big[:, :32] == -5) and torch.all(big[:, 32 + N:] == -5)


# --- pins on the GPU ------------------------------------------------------------------------

def test_integer_valued_fp16_is_exact(lib):
    """Integers in [-8, 8]: every partial sum is an integer below 2^24, so any
    FP32 summation order is exact and the result must equal the oracle."""
    for (M, N, K) in [(1024, 1024, 1024), (512, 768, 640), (300, 290, 333)]:
        A, B = _operands(F16, M, N, K, seed=M + 2 * N, dist="int")
        dA, dB = to_device(A), to_device(B)
        for kind in ("single", "pipelined"):
            check_f16(gemm(lib, F16, kind, dA, dB), A, B, exact=True)


@pytest.mark.parametrize("M,N,K,which", [(256, 192, 512, "A"), (192, 256, 512, "B"),
                                          (130, 70, 16, "both")])
def test_fp16_subnormal_inputs_are_exact(lib, M, N, K, which):
    """binary16 subnormals (m * 2^-24) against small integers, or against each
    other at small K: every product and partial sum is an integer multiple of
    2^-24 (2^-48) below 2^24 units, so FP32 holds it exactly in any order and
    the result must equal the oracle bit for bit.  A flush of subnormal
    inputs to zero fails this."""
    sub_a = which in ("A", "both")
    sub_b = which in ("B", "both")
    A = si.f16_subnormals(M, K, seed=M + K) if sub_a else si.f16_integers(M, K, seed=M + K)
    B = si.f16_subnormals(K, N, seed=N + K) if sub_b else si.f16_integers(K, N, seed=N + K)
    dA, dB = to_device(A), to_device(B)
    for kind in ("single", "pipelined"):
        C = gemm(lib, F16, kind, dA, dB)
        check_f16(C, A, B, exact=True)
        assert C.abs().max().item() > 0


def test_integer_valued_fp32_is_exact(lib):
    """The same pin for FP32 inputs: layout and indexing with no tolerance."""
    for (M, N, K) in [(1024, 1024, 1024), (512, 768, 640), (300, 288, 336), (300, 290, 333)]:
        A, B = _operands(F32, M, N, K, seed=M + 3 * N, dist="int")
        dA, dB = to_device(A), to_device(B)
        for kind in ("single", "pipelined"):
            check_f32(gemm(lib, F32, kind, dA, dB), A, B, exact=True)


def test_exhaustive_int8_product_table(lib):
    vals = np.arange(-128, 128, dtype=np.int16).astype(np.int8)
    A = vals.reshape(256, 1).copy()
    B = vals[::-1].reshape(1, 256).copy()
    for kind in ("single", "pipelined"):
        check_i8(gemm(lib, I8, kind, to_device(A), to_device(B)), A, B)


@pytest.mark.parametrize("dtype", [F16, I8, F32])
def test_identity(lib, dtype):
    n = 512
    A, _ = _operands(dtype, n, n, n, seed=21)
    if dtype == F16:
        one = np.float16(1.0).view(np.uint16)
        I = np.where(np.eye(n, dtype=bool), one, np.uint16(0)).astype(np.uint16)
        expect = A.view(np.float16).astype(np.float32)
    elif dtype == F32:
        I = np.eye(n, dtype=np.float32)
        expect = A
    else:
        I = np.eye(n, dtype=np.int8)
        expect = A.astype(np.int32)
    dA, dI = to_device(A), to_device(I)
    for kind in ("single", "pipelined"):
        assert np.array_equal(gemm(lib, dtype, kind, dA, dI).cpu().numpy(), expect)
        assert np.array_equal(gemm(lib, dtype, kind, dI, dA).cpu().numpy(),
                              expect if dtype == I8 else expect)


def test_rank1_extremes_int8(lib):
    """A[i][k] = u_i, B[k][j] = v_j: C = K u_i v_j, up to 4096 * 16384."""
    M, N, K = 512, 512, 4096
    u = np.resize(np.array([-128, 127, 1, -1, 0, 64, -64, 5], dtype=np.int8), M)
    v = np.resize(np.array([127, -128, -1, 1, 3, 0, 100, -7], dtype=np.int8), N)
    A = np.repeat(u.reshape(M, 1), K, axis=1)
    B = np.repeat(v.reshape(1, N), K, axis=0)
    expect = K * np.outer(u.astype(np.int64), v.astype(np.int64))
    for kind in ("single", "pipelined"):
        got = gemm(lib, I8, kind, to_device(A), to_device(B)).cpu().numpy()
        assert np.array_equal(got.astype(np.int64), expect)


def test_all_ones_detects_a_dropped_tile(lib):
    """All-ones operands give C = K everywhere; a lost K tile would give K - BK."""
    import torch
    M, N, K = 512, 512, 1024
    for dtype in (F16, I8, F32):
        if dtype == F16:
            A = np.full((M, K), np.float16(1.0).view(np.uint16), dtype=np.uint16)
            B = np.full((K, N), np.float16(1.0).view(np.uint16), dtype=np.uint16)
        elif dtype == F32:
            A = np.ones((M, K), dtype=np.float32)
            B = np.ones((K, N), dtype=np.float32)
        else:
            A = np.ones((M, K), dtype=np.int8)
            B = np.ones((K, N), dtype=np.int8)
        for kind in ("single", "pipelined"):
            C = gemm(lib, dtype, kind, to_device(A), to_device(B))
            assert torch.all(C == K)


def test_k_split_additivity(lib):
    """C(A, B) == C(A[:, :k1], B[:k1]) + C(A[:, k1:], B[k1:]) exactly for INT8,
    with the halves passed as pointer offsets into the same matrices."""
    import torch
    M, N, K = 512, 512, 1024
    A, B = _operands(I8, M, N, K, seed=31)
    dA, dB = to_device(A), to_device(B)
    full = gemm(lib, I8, "pipelined", dA, dB)
    for k1 in (128, 384, 512):
        part = gemm(lib, I8, "pipelined", dA[:, :k1], dB[:k1]) + \
            gemm(lib, I8, "pipelined", dA[:, k1:], dB[k1:])
        assert torch.equal(full, part)


@pytest.mark.parametrize("name,launches", [("fp16_1024", 10), ("fp16_4096", 60), ("int8_4096", 60),
                                           ("fp16_skinny", 60)])
def test_repeat_runs_are_bitwise_identical(lib, name, launches):
    """The benchmark's workloads launched one after another with no host
    wait between them, into alternating outputs: every launch equals the
    first bit for bit (compared on the device, in stream order).  A missing
    wait or barrier in the K loop lets a launch read a tile before it lands,
    and shows up here as a launch that differs."""
    import torch
    wl = si.WORKLOADS[name]
    A, B = wl.operands()
    dA, dB = to_device(A), to_device(B)
    dt = I8 if wl.dtype == "i8" else F16
    first = gemm(lib, dt, "pipelined", dA, dB)
    outs = [torch.empty_like(first) for _ in range(2)]
    differs = []
    for i in range(launches):
        C = outs[i % 2]
        C.fill_(-1)
        gemm(lib, dt, "pipelined", dA, dB, C)
        differs.append(torch.ne(C, first).any())
    bad = [i for i, d in enumerate(differs) if bool(d)]
    assert not bad, (name, bad)


def test_concurrent_streams_from_host_threads(lib):
    """Four host threads, each on a stream of its own, launch products of
    different dtypes and shapes at the same time (the plan cache is shared);
    every result matches the oracle and repeats bit for bit."""
    import threading
    import torch
    cases = [(F16, 512, 384, 640), (I8, 300, 290, 333), (F32, 256, 320, 256), (F16, 1000, 70, 129)]
    host = [_operands(dt, M, N, K, seed=40 + i) for i, (dt, M, N, K) in enumerate(cases)]
    dev = [(to_device(A), to_device(B)) for A, B in host]
    torch.cuda.synchronize()
    results, errors = [None] * len(cases), []

    def worker(i):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                outs = [gemm(lib, cases[i][0], "pipelined", *dev[i]) for _ in range(6)]
            stream.synchronize()
            results[i] = outs
        except Exception as exc:  # reported below, in the main thread
            errors.append(exc)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for (dt, M, N, K), (A, B), outs in zip(cases, host, results):
        _check(dt, outs[0], A, B)
        for C in outs[1:]:
            assert torch.equal(C, outs[0])


@pytest.mark.parametrize("dtype,M,N,K", [(F16, 2048, 64, 8192), (I8, 2048, 64, 8192),
                                         (F32, 1024, 64, 4096), (F16, 1000, 70, 4000),
                                         (I8, 777, 100, 5000), (F16, 512, 512, 1024),
                                         # bounds-checked DMA: the partial K tile sits at a
                                         # different walk position in every tile row
                                         (F16, 1000, 72, 4000), (I8, 777, 112, 5008),
                                         (F32, 500, 68, 3000)])
def test_k_rotation_against_the_plain_walk(lib, dtype, M, N, K):
    """Shapes whose B fits in L2 walk K from a per-tile-row offset.  The
    same call with the rotation switched off (debug flag) walks K from 0:
    both match the oracle, INT8 bit for bit (and the sequential entry point
    too), so only the summation order differs.  The loop forms' bitwise
    agreement under the rotation is what test_tile_shape_all_variants checks
    (its shapes all rotate)."""
    import torch
    _, info = lib.tdg_plan(CODE[dtype], M, N, K)
    assert info["k_rotated"] == 1
    A, B = _operands(dtype, M, N, K, seed=M + 3 * K)
    dA, dB = to_device(A), to_device(B)
    rotated = gemm(lib, dtype, "pipelined", dA, dB)
    prev = lib.tdg_set_debug_flags(lib.TDG_DEBUG_NO_K_ROTATION)
    try:
        plain = gemm(lib, dtype, "pipelined", dA, dB)
    finally:
        lib.tdg_set_debug_flags(prev)
    _check(dtype, rotated, A, B)
    _check(dtype, plain, A, B)
    if dtype == I8:
        assert torch.equal(rotated, plain)
        assert torch.equal(rotated, gemm(lib, dtype, "single", dA, dB))


@pytest.mark.parametrize("dtype", [F16, I8, F32])
@pytest.mark.parametrize("M,N,K,parts", [(256, 256, 8192, 0), (256, 256, 8192, 1), (256, 256, 8192, 7),
                                         (130, 70, 3000, 5),
                                         (300, 290, 4099, 3), (64, 64, 65536, 0), (512, 384, 2048, 2),
                                         (100, 100, 600, 64)])
def test_split_k(lib, dtype, M, N, K, parts):
    """K split over `parts` workgroups per tile (0: the planner's choice; 1:
    the plain product, equal to the pipelined call bit for bit; a count above
    the K tiles is lowered), partial tiles summed in part order: against the
    oracle, bitwise repeatable, INT8 equal to the unsplit call; once more
    under the LDS poisoning race screen."""
    import torch
    A, B = _operands(dtype, M, N, K, seed=M + 5 * K + parts)
    dA, dB = to_device(A), to_device(B)
    fn = {F16: lib.gemm_f16f32_splitk, I8: lib.gemm_i8i32_splitk, F32: lib.gemm_f32f32_splitk}[dtype]
    C1 = fn(dA, dB, parts=parts)
    _check(dtype, C1, A, B)
    assert torch.equal(C1, fn(dA, dB, parts=parts))
    if dtype == I8 or parts == 1:
        assert torch.equal(C1, gemm(lib, dtype, "pipelined", dA, dB))
    prev = lib.tdg_set_debug_flags(lib.TDG_DEBUG_POISON_LDS)
    try:
        C2 = fn(dA, dB, parts=parts)
    finally:
        lib.tdg_set_debug_flags(prev)
    assert torch.equal(C1, C2)


@pytest.mark.parametrize("dtype", [F16, I8, F32])
def test_split_k_with_an_empty_k_zero_fills(lib, dtype):
    """K = 0 through the split-K entry points with the part count left to
    the planner (parts = 0, straight through the C ABI) and through the
    allocation-free one: C is all zeros."""
    import torch
    lib_c = lib.load_library()
    out_t = torch.int32 if dtype == I8 else torch.float32
    raw = {F16: lib_c.gemm_f16f32_splitk, I8: lib_c.gemm_i8i32_splitk, F32: lib_c.gemm_f32f32_splitk}[dtype]
    in_t = {F16: torch.float16, I8: torch.int8, F32: torch.float32}[dtype]
    for M, N in ((64, 1), (300, 260)):
        C = torch.full((M, N), 7, dtype=out_t, device="cuda")
        stream = torch.cuda.current_stream().cuda_stream
        assert raw(M, N, 0, None, 1, None, N, C.data_ptr(), N, 0, None, 0, stream) == lib.TDG_OK
        torch.cuda.synchronize()
        assert torch.count_nonzero(C).item() == 0, (M, N)
        C.fill_(7)
        A = torch.empty((M, 0), dtype=in_t, device="cuda")
        B = torch.empty((0, N), dtype=in_t, device="cuda")
        lib.gemm_splitk_noalloc(A, B, C, parts=0)
        torch.cuda.synchronize()
        assert torch.count_nonzero(C).item() == 0, (M, N)


def test_split_k_strided_output_and_explicit_workspace(lib):
    """Split K into a strided C view, through a caller-given workspace with
    room to spare; C's padding stays untouched."""
    import torch
    M, N, K, P = 200, 136, 5000, 6
    A, B = _operands(F16, M, N, K, seed=99)
    big = torch.full((M, N + 9), -2.0, dtype=torch.float32, device="cuda")
    C = big[:, 3:3 + N]
    ws = torch.empty(P * M * N * 4 + 4096, dtype=torch.uint8, device="cuda")
    lib.gemm_f16f32_splitk(to_device(A), to_device(B), C, parts=P, workspace=ws)
    check_f16(C, A, B)
    assert torch.all(big[:, :3] == -2.0) and torch.all(big[:, 3 + N:] == -2.0)


def test_invalid_arguments_are_rejected(lib):
    import torch
    A = torch.zeros((64, 64), dtype=torch.int8, device="cuda")
    B = torch.zeros((64, 64), dtype=torch.int8, device="cuda")
    buf = torch.zeros((64 * 64,), dtype=torch.int32, device="cuda")
    p = buf.data_ptr()
    # C overlapping A
    assert lib.call_raw("gemm_i8i32_pipelined", 16, 16, 16, p, 16, B.data_ptr(), 64, p, 16) == \
        lib.TDG_ERR_INVALID_ARG
    # lda too small
    assert lib.call_raw("gemm_i8i32", 64, 64, 64, A.data_ptr(), 32, B.data_ptr(), 64, p, 64) == \
        lib.TDG_ERR_INVALID_ARG
    # explicit tile that is not built
    cfg = lib.TdgConfig(bm=96, bn=96, bk=0, waves=0, lds_stages=0, variant=0)
    assert lib.call_raw("gemm_i8i32_ex", 64, 64, 64, A.data_ptr(), 64, B.data_ptr(), 64, p, 64,
                        0, cfg) == lib.TDG_ERR_UNSUPPORTED


def test_binding_rejects_host_tensors(lib):
    """The binding passes device pointers only: an output, workspace or
    copy destination in host memory is refused before the library is
    called, and the output is left as it was."""
    import torch
    A = torch.ones((64, 64), dtype=torch.float16, device="cuda")
    B = torch.ones((64, 64), dtype=torch.float16, device="cuda")
    host_C = torch.full((64, 64), 7.0)
    with pytest.raises(ValueError):
        lib.gemm_f16f32_pipelined(A, B, host_C)
    assert torch.all(host_C == 7.0)
    with pytest.raises(ValueError):
        lib.gemm_f16f32_pipelined(A.cpu(), B)
    with pytest.raises(ValueError):
        lib.gemm_f16f32_splitk(A, B, parts=2, workspace=torch.empty(2 * 64 * 64 * 4, dtype=torch.uint8))
    ws = torch.empty(4 * 64 * 64 * 4, dtype=torch.uint8, device="cuda")[::2]  # not contiguous
    with pytest.raises(ValueError):
        lib.gemm_f16f32_splitk(A, B, parts=2, workspace=ws)
    with pytest.raises(ValueError):  # the C ABI answers TDG_ERR_INVALID_ARG; the binding says so first
        lib.gemm_f16f32_splitk(A, B, parts=-1)
    x = torch.ones((64, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        lib.tdg_transpose_f32(x, out=torch.empty((64, 64)))
    torch.cuda.synchronize()


# --- the full-size workloads, in the configuration the benchmark times: whole outputs ------

@pytest.mark.parametrize("name", ["int8_4096", "fp16_4096", "fp16_skinny", "fp32_4096", "fp16_shard8",
                                  "int8_shard8"])
def test_full_size_whole_output(lib, name):
    """The benchmark's workloads in the configuration it times: every element
    of C against the oracle (INT8 bit for bit, FP16 / FP32 within
    1e-4 * sum |a b| and within the pages' own absolute / relative pair),
    after a quick check of sampled elements (tile corners included) that
    gives an early, readable failure.  The sequential loop and
    every other built loop form at the planner's tile must then equal the
    pipelined output bit for bit ("Pipeline GPU Kernel", Step 5: check a small
    size, then the target size, against the CPU reference)."""
    import torch
    wl = si.WORKLOADS[name]
    A, B = wl.operands()
    dA, dB = to_device(A), to_device(B)
    dtype = {"i8": I8, "f16": F16, "f32": F32}[wl.dtype]
    rows, cols = sample_indices(wl.M, wl.N, 3000, seed=wl.seed_a, tile_n=min(256, wl.N))
    C_pipe = gemm(lib, dtype, "pipelined", dA, dB)
    check_sampled(C_pipe, dtype, A, B, rows, cols)
    _check(dtype, C_pipe, A, B, pages_rule=True)
    C_single = gemm(lib, dtype, "single", dA, dB)
    assert torch.equal(C_pipe, C_single)
    tile, _ = lib.tdg_plan(CODE[dtype], wl.M, wl.N, wl.K)
    for vname, cfg in _variants(lib, dtype, tile):
        assert torch.equal(C_pipe, gemm(lib, dtype, "ex", dA, dB, cfg=cfg)), vname
    del C_pipe, C_single, dA, dB
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype,M,N,K", [(F16, 4095, 4095, 4095), (I8, 4097, 4097, 4097),
                                         (F32, 4095, 4095, 4095)])
def test_large_odd_whole_output(lib, dtype, M, N, K):
    """Odd sizes near the benchmark sizes: most rows start off a 16-byte
    boundary, and the planner keeps the bounds-checked direct-to-LDS loop
    (or, when an operand's last chunk would leave its page, the
    bounds-checked register-prefetch loop); every element against the
    oracle (sampled tile edges first, for an early failure message), and
    the whole output bit for bit against the guarded sequential and
    register-prefetch loops."""
    import torch
    A, B = _operands(dtype, M, N, K, seed=M + 7)
    dA, dB = to_device(A), to_device(B)
    code = CODE[dtype]
    cfg, info = lib.tdg_plan_operands(code, M, N, K, dA.data_ptr(), dA.stride(0), dB.data_ptr(),
                                      dB.stride(0))
    assert info["guarded"] == 1
    assert cfg["variant"] in (lib.TDG_VARIANT_DIRECT_LDS, lib.TDG_VARIANT_REG_PREFETCH)
    rows, cols = sample_indices(M, N, 2000, seed=M, tile_m=cfg["bm"], tile_n=cfg["bn"])
    C = gemm(lib, dtype, "pipelined", dA, dB)
    check_sampled(C, dtype, A, B, rows, cols)
    _check(dtype, C, A, B)
    single = dict(cfg, variant=lib.TDG_VARIANT_SINGLE, lds_stages=1)
    assert torch.equal(C, gemm(lib, dtype, "ex", dA, dB, cfg=single))
    reg = dict(cfg, variant=lib.TDG_VARIANT_REG_PREFETCH, lds_stages=2)
    assert torch.equal(C, gemm(lib, dtype, "ex", dA, dB, cfg=reg))
    del C, dA, dB
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", [F16, I8, F32])
def test_large_split_chunk_whole_output(lib, dtype):
    """4095^3 stored with leading dimensions 4096 (rows 16-byte aligned, K
    and N ending inside a chunk, NaN / 127 in the padding column): the
    planner keeps the bounds-checked direct-to-LDS loop; every element
    against the oracle and the whole output bit for bit against the guarded
    register-prefetch loop."""
    import torch
    M = N = K = 4095
    A, B, dA, dB = _split_chunk_operands(dtype, M, N, K, seed=4095 + 11, pad_chunks=0)
    assert dA.stride(0) == 4096 and dB.stride(0) == 4096
    code = CODE[dtype]
    cfg, info = lib.tdg_plan(code, M, N, K)
    C = gemm(lib, dtype, "pipelined", dA, dB)
    rows, cols = sample_indices(M, N, 2000, seed=M, tile_m=cfg["bm"], tile_n=cfg["bn"])
    check_sampled(C, dtype, A, B, rows, cols)
    _check(dtype, C, A, B)
    reg = dict(cfg, variant=lib.TDG_VARIANT_REG_PREFETCH, lds_stages=2)
    assert torch.equal(C, gemm(lib, dtype, "ex", dA, dB, cfg=reg))
    del C, dA, dB
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype,M,N,K", [(F16, 4000, 4000, 4000), (I8, 4000, 4000, 4000),
                                         (F16, 16383, 64, 8184), (F32, 4000, 4000, 4000)])
def test_large_ragged_whole_output(lib, dtype, M, N, K):
    """Ragged shapes near the benchmark sizes run the bounds-checked
    direct-to-LDS loop; every element against the oracle (sampled tile edges
    first), and the whole output against the guarded register-prefetch loop
    bit for bit."""
    import torch
    A, B = _operands(dtype, M, N, K, seed=M + K)
    dA, dB = to_device(A), to_device(B)
    code = CODE[dtype]
    cfg, info = lib.tdg_plan(code, M, N, K)
    assert info["guarded"] == 1 and cfg["variant"] == lib.TDG_VARIANT_DIRECT_LDS
    rows, cols = sample_indices(M, N, 2000, seed=M, tile_m=cfg["bm"], tile_n=min(cfg["bn"], N))
    C = gemm(lib, dtype, "pipelined", dA, dB)
    check_sampled(C, dtype, A, B, rows, cols)
    _check(dtype, C, A, B)
    reg = dict(cfg, variant=lib.TDG_VARIANT_REG_PREFETCH, lds_stages=2)
    assert torch.equal(C, gemm(lib, dtype, "ex", dA, dB, cfg=reg))
    del C, dA, dB
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", [F16, I8, F32])
def test_graph_capture_replays(lib, dtype):
    """The pipelined entry point captured in a HIP graph: every replay, with
    new operand values copied in between, matches the oracle and the eager
    call."""
    import torch
    M, N, K = 512, 384, 320
    dA = to_device(_operands(dtype, M, N, K, seed=50)[0])
    dB = to_device(_operands(dtype, M, N, K, seed=50)[1])
    out_t = torch.int32 if dtype == I8 else torch.float32
    C = torch.zeros((M, N), dtype=out_t, device="cuda")
    gemm(lib, dtype, "pipelined", dA, dB, C)   # first call outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gemm(lib, dtype, "pipelined", dA, dB, C)
    for rep in range(3):
        A, B = _operands(dtype, M, N, K, seed=60 + rep)
        dA.copy_(to_device(A))
        dB.copy_(to_device(B))
        C.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _check(dtype, C, A, B)
        eager = gemm(lib, dtype, "pipelined", dA, dB)
        assert torch.equal(C, eager)


# --- maximum sizes ----------------------------------------------------------------------

@pytest.mark.parametrize("K", [131071, 131056])
def test_int8_largest_k_without_overflow(lib, K):
    """All inputs -128: C = 16384 * K, the largest INT32 sum the method can
    produce at this K (131071 is the last K below 2^31 / 2^14).  K = 131071
    runs the element-wise guarded loop, 131056 (whole 16-byte chunks) the
    bounds-checked direct-to-LDS loop."""
    import torch
    M, N = 64, 80
    A = np.full((M, K), -128, dtype=np.int8)
    B = np.full((K, N), -128, dtype=np.int8)
    for kind in ("single", "pipelined"):
        C = gemm(lib, I8, kind, to_device(A), to_device(B))
        assert torch.all(C == 16384 * K), kind
    assert 16384 * 131071 < 2 ** 31


def test_fp16_long_k_exact(lib):
    """K = 131072 with +-1 inputs: every partial sum is an integer below 2^24,
    so FP32 accumulation is exact in any order; the oracle decides."""
    M, N, K = 64, 64, 131072
    rng = np.random.default_rng(77)
    A = np.where(rng.random((M, K)) < 0.5, np.float16(-1.0), np.float16(1.0)).astype(np.float16)
    B = np.where(rng.random((K, N)) < 0.5, np.float16(-1.0), np.float16(1.0)).astype(np.float16)
    A, B = A.view(np.uint16), B.view(np.uint16)
    for kind in ("single", "pipelined"):
        check_f16(gemm(lib, F16, kind, to_device(A), to_device(B)), A, B, exact=True)


def test_tall_grid(lib):
    """M = 2^20 rows, N = 64: 16384 workgroups; every element against the
    oracle (sampled rows first), and the whole output against the sequential
    loop bit for bit."""
    import torch
    M, N, K = 1 << 20, 64, 128
    A, B = _operands(F16, M, N, K, seed=88)
    dA, dB = to_device(A), to_device(B)
    C = gemm(lib, F16, "pipelined", dA, dB)
    rows, cols = sample_indices(M, N, 4000, seed=88, tile_m=64, tile_n=64)
    check_sampled(C, F16, A, B, rows, cols)
    check_f16(C, A, B)
    assert torch.equal(C, gemm(lib, F16, "single", dA, dB))


def test_row_panel_shard_is_the_full_products_rows(lib):
    """Split by C row panels, GPU 0's share (512 x 4096 x 4096) needs no
    exchange: its INT8 product equals rows 0..511 of the full 4096^3 product
    bit for bit, whatever tile each size is planned with."""
    import torch
    full, shard = si.WORKLOADS["int8_4096"], si.WORKLOADS["int8_shard8"]
    A, B = full.operands()
    As, Bs = shard.operands()
    assert np.array_equal(As, A[:512]) and np.array_equal(Bs, B)
    dA, dB = to_device(A), to_device(B)
    C_full = gemm(lib, I8, "pipelined", dA, dB)
    C_shard = gemm(lib, I8, "pipelined", to_device(As), dB)
    torch.cuda.synchronize()
    assert torch.equal(C_shard, C_full[:512])


def test_binding_launches_on_the_current_stream(lib):
    """The binding passes torch's current stream: the raw handle it reads
    equals torch.cuda.current_stream().cuda_stream, also inside a side
    stream's context, and a product enqueued there is complete after that
    stream alone is synchronised."""
    import torch
    from tiled_dense_gemm_loop_amd import _binding as b
    dev = torch.cuda.current_device()
    assert b._stream_handle(dev) == torch.cuda.current_stream().cuda_stream
    A8, B8 = si.i8_uniform(256, 256, 61), si.i8_uniform(256, 256, 62)
    dA, dB = to_device(A8), to_device(B8)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        assert b._stream_handle(dev) == side.cuda_stream
        assert b._stream_handle(dev) != torch.cuda.default_stream().cuda_stream
        C = lib.gemm_i8i32_pipelined(dA, dB)
    side.synchronize()
    assert np.array_equal(C.cpu().numpy().astype(np.int64), oracle.gemm_i8(A8, B8))
