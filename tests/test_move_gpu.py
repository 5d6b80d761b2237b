"""GPU parity of the copy / transpose ladder ("fixing GPU kernels by hand",
the transpose exercise) against the CPU oracle: every method moves 32-bit
patterns, so the result must match bit for bit -- NaN payloads, signed zeros
and subnormals included."""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

METHODS = ["naive", "lds", "lds_padded", "lds_swizzled", "vec"]
SHAPES = [(1, 1), (1, 64), (64, 1), (7, 13), (64, 64), (65, 63), (63, 65), (128, 256),
          (300, 500), (1000, 37), (4096, 4096)]


@pytest.fixture(scope="module")
def lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import tiled_dense_gemm_loop_amd as t
    t.load_library()
    return t


def _bits(rows, cols, seed):
    x = np.random.default_rng(seed).integers(0, 2 ** 32, size=(rows, cols), dtype=np.uint64)
    x = x.astype(np.uint32)
    if x.size:
        x.flat[::97] = 0x7FC01234   # NaN with a payload
        x.flat[1::89] = 0x80000000  # -0.0
        x.flat[2::83] = 0x00000003  # subnormal
    return x


def _dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int32)).cuda().view(torch.float32)


def _host(t):
    import torch
    return t.view(torch.int32).cpu().numpy().view(np.uint32)


def _method(lib, name):
    return getattr(lib, "TDG_TRANSPOSE_" + name.upper())


@pytest.mark.parametrize("rows,cols", SHAPES)
def test_copy_bit_exact(lib, rows, cols):
    x = _bits(rows, cols, rows * 7 + cols)
    got = _host(lib.tdg_copy_f32(_dev(x)))
    assert np.array_equal(got, oracle.copy_u32(x))


@pytest.mark.parametrize("method", METHODS)
@pytest.mark.parametrize("rows,cols", SHAPES)
def test_transpose_bit_exact(lib, method, rows, cols):
    x = _bits(rows, cols, rows * 11 + cols)
    got = _host(lib.tdg_transpose_f32(_dev(x), method=_method(lib, method)))
    ref = oracle.transpose_u32(x)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, "%d mismatches, first at %s" % (len(bad), tuple(bad[0]))


@pytest.mark.parametrize("method", METHODS + ["copy"])
def test_strided_and_misaligned(lib, method):
    """Row strides wider than the matrix on both sides, and bases that are
    not 16-byte aligned (the vector form must fall back); padding of the
    output stays untouched."""
    import torch
    rows, cols = 200, 136
    big = _bits(rows + 3, cols + 20, 5)
    for off in (0, 1):
        x_host = big[2:2 + rows, off:off + cols]
        dx = _dev(big)[2:2 + rows, off:off + cols]
        orows, ocols = (rows, cols) if method == "copy" else (cols, rows)
        out_big = torch.full((orows, ocols + 12), -7.0, dtype=torch.float32, device="cuda")
        out = out_big[:, off:off + ocols]
        if method == "copy":
            lib.tdg_copy_f32(dx, out)
            ref = oracle.copy_u32(x_host)
        else:
            lib.tdg_transpose_f32(dx, out, method=_method(lib, method))
            ref = oracle.transpose_u32(x_host)
        assert np.array_equal(_host(out), ref)
        pad = out_big.cpu().numpy()
        assert np.all(pad[:, :off] == -7.0) and np.all(pad[:, off + ocols:] == -7.0)


def test_every_method_agrees_and_involution(lib):
    rows, cols = 1111, 777
    x = _bits(rows, cols, 3)
    dx = _dev(x)
    outs = [_host(lib.tdg_transpose_f32(dx, method=_method(lib, m))) for m in METHODS]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    back = lib.tdg_transpose_f32(lib.tdg_transpose_f32(dx))
    assert np.array_equal(_host(back), x)


def test_large_matrix_blocks(lib):
    """16384 x 16384 (1 GiB each way, well beyond the 256 MB last-level
    cache): blocks at the corners, tile edges and random spots against the
    oracle's transpose of the same input blocks."""
    import torch
    n = 16384
    gen = torch.Generator(device="cuda").manual_seed(1234)
    dx = torch.randint(-2 ** 31, 2 ** 31 - 1, (n, n), dtype=torch.int32, device="cuda",
                       generator=gen).view(torch.float32)
    rng = np.random.default_rng(0)
    starts = [(0, 0), (n - 96, n - 96), (64 * 100 - 16, 64 * 37 - 16)] + \
        [tuple(int(v) for v in rng.integers(0, n - 96, 2)) for _ in range(5)]
    for method in ["copy"] + METHODS:
        if method == "copy":
            out = lib.tdg_copy_f32(dx)
        else:
            out = lib.tdg_transpose_f32(dx, method=_method(lib, method))
        for (r, c) in starts:
            blk = _host(dx[r:r + 96, c:c + 96])
            if method == "copy":
                assert np.array_equal(_host(out[r:r + 96, c:c + 96]), oracle.copy_u32(blk))
            else:
                assert np.array_equal(_host(out[c:c + 96, r:r + 96]), oracle.transpose_u32(blk))
        del out
    del dx
    torch.cuda.empty_cache()


def test_random_shapes_strides_and_offsets(lib):
    """A seeded sweep: random shapes (1..1500, a third near multiples of the
    64-wide tile), input and output views at element offsets 0..5 with row
    padding 0..9, every method and the copy, each against the oracle bit for
    bit; the output's padding stays untouched."""
    import random
    import torch
    rng = random.Random(21)
    methods = ["copy"] + METHODS + ["auto"]
    for case in range(60):
        rows, cols = rng.randint(1, 1500), rng.randint(1, 1500)
        if rng.random() < 0.3:
            rows = max(1, rng.choice((64, 128, 256, 1024)) + rng.randint(-2, 2))
            cols = max(1, rng.choice((64, 128, 256, 1024)) + rng.randint(-2, 2))
        oi, pi, oo, po = rng.randint(0, 5), rng.randint(0, 9), rng.randint(0, 5), rng.randint(0, 9)
        big = _bits(rows, cols + oi + pi, 700 + case)
        x = big[:, oi:oi + cols]
        dx = _dev(big)[:, oi:oi + cols]
        m = rng.choice(methods)
        orows, ocols = (rows, cols) if m == "copy" else (cols, rows)
        out_big = torch.full((orows, ocols + oo + po), -7.0, dtype=torch.float32, device="cuda")
        out = out_big[:, oo:oo + ocols]
        if m == "copy":
            lib.tdg_copy_f32(dx, out)
            ref = oracle.copy_u32(x)
        else:
            lib.tdg_transpose_f32(dx, out, method=_method(lib, m))
            ref = oracle.transpose_u32(x)
        what = (case, rows, cols, oi, pi, oo, po, m)
        assert np.array_equal(_host(out), ref), what
        pad = out_big.cpu().numpy()
        assert np.all(pad[:, :oo] == -7.0) and np.all(pad[:, oo + ocols:] == -7.0), what
