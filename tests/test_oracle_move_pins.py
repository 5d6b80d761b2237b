"""Pins for the copy / transpose oracle ("fixing GPU kernels by hand", the
four-step transpose exercise), each against something other than itself:
numpy's own transpose and copy, the involution T(T(x)) = x, index-encoded
matrices whose every element names its own position, and bit patterns that
arithmetic would alter (NaN payloads, signed zeros, subnormals).  The last
test plants a plausible slip (the output leading dimension of a non-square
transpose taken from the wrong side) and shows the pins catch it."""
import ctypes

import numpy as np
import pytest

import oracle

SHAPES = [(1, 1), (1, 7), (7, 1), (3, 5), (64, 64), (65, 63), (100, 37), (256, 300), (0, 5), (5, 0)]


def _bits(rows, cols, seed):
    return np.random.default_rng(seed).integers(0, 2 ** 32, size=(rows, cols), dtype=np.uint64) \
        .astype(np.uint32)


@pytest.mark.parametrize("rows,cols", SHAPES)
def test_transpose_matches_numpy(rows, cols):
    x = _bits(rows, cols, rows * 1000 + cols)
    assert np.array_equal(oracle.transpose_u32(x), x.T)


@pytest.mark.parametrize("rows,cols", SHAPES)
def test_copy_matches_numpy(rows, cols):
    x = _bits(rows, cols, rows * 999 + cols)
    got = oracle.copy_u32(x)
    assert got.shape == x.shape and np.array_equal(got, x)


@pytest.mark.parametrize("rows,cols", [(3, 5), (65, 63), (128, 200)])
def test_transpose_is_an_involution(rows, cols):
    x = _bits(rows, cols, 5)
    assert np.array_equal(oracle.transpose_u32(oracle.transpose_u32(x)), x)


def test_index_encoded_positions():
    """Element (i, j) holds i * 2^16 + j: after the transpose the element at
    (a, b) must name position (b, a)."""
    rows, cols = 300, 257
    i, j = np.meshgrid(np.arange(rows, dtype=np.uint32), np.arange(cols, dtype=np.uint32),
                       indexing="ij")
    x = (i << 16) | j
    t = oracle.transpose_u32(x)
    a, b = np.meshgrid(np.arange(cols), np.arange(rows), indexing="ij")
    assert np.array_equal(t >> 16, b) and np.array_equal(t & 0xFFFF, a)


def test_strided_input_rows():
    big = _bits(40, 90, 9)
    view = big[3:33, 10:70]            # leading dimension 90, not 60
    assert np.array_equal(oracle.transpose_u32(view), view.T)
    assert np.array_equal(oracle.copy_u32(view), view)


def test_bit_patterns_survive():
    specials = np.array([0x7FC00001, 0xFFC12345, 0x7F800001, 0x80000000, 0x00000001, 0x807FFFFF,
                         0x7F800000, 0xFF800000, 0x3F800000, 0x00000000], dtype=np.uint32)
    x = np.resize(specials, (10, 13))
    assert np.array_equal(oracle.transpose_u32(x).T, x)
    assert np.array_equal(oracle.copy_u32(x.view(np.float32)), x)


def test_invalid_arguments_rejected():
    lib = oracle._load()
    buf = np.zeros(16, dtype=np.uint32)
    p = buf.ctypes.data
    assert lib.oracle_transpose_u32(4, 4, p, 3, p, 4) == -1   # ldi < cols
    assert lib.oracle_transpose_u32(3, 4, p, 4, p, 2) == -1   # ldo < rows
    assert lib.oracle_copy_u32(-1, 4, p, 4, p, 4) == -1
    assert lib.oracle_copy_u32(2, 2, None, 2, p, 2) == -1


def test_pins_catch_a_wrong_output_leading_dimension():
    """A transpose that strides its output by the input's row length (cols)
    instead of the output's (rows) agrees on square matrices and fails the
    numpy pin on a non-square one."""
    lib = oracle._load()

    def wrong(x):
        rows, cols = x.shape
        out = np.zeros(cols * max(rows, cols), dtype=np.uint32)
        assert lib.oracle_transpose_u32(rows, cols, x.ctypes.data, cols, out.ctypes.data, cols) == 0
        return out[:cols * rows].reshape(cols, rows)   # read back as a dense cols x rows matrix

    sq = _bits(20, 20, 1)
    assert np.array_equal(wrong(sq), sq.T)
    ns = _bits(12, 20, 2)
    assert not np.array_equal(wrong(ns), ns.T)
