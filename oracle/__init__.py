"""The plain CPU oracle for C = A.B (FP16 -> FP64 reference, INT8 -> INT64).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark are the only callers.  The GPU library never imports,
links or runs anything in this directory, and this directory never imports the
GPU library.

The arithmetic lives in ``oracle_gemm.c`` and ``oracle_move.c`` (plain C,
built with gcc); this module only builds them and marshals numpy arrays into
them.  What it computes is
the textbook product, C[i][j] = sum_k A[i][k] * B[k][j] in increasing k, in
int64 for INT8 inputs and in double for binary16 and binary32 inputs (each
input widened exactly), with S[i][j] = sum_k |A[i][k] * B[k][j]| beside the
floating-point results.
("Pipeline GPU Kernel", Step 2 and Step 5; "Analyze Kernel Bottleneck",
Step 1.)

Pins (tests/test_oracle_pins.py) tie it to things other than itself: brute
force with Python integers and exact fractions, the exhaustive int8 product
table, identity and rank-1 closed forms, K-split additivity, the transpose
identity, numpy's matmul in int64/float64, and numpy's own binary16 widening.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_gemm.c")
_SRC_MOVE = os.path.join(_HERE, "oracle_move.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_gemm.so")
_lib = None


def build() -> str:
    """Compile oracle_gemm.c and oracle_move.c into liboracle_gemm.so with gcc
    (no fast-math)."""
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-D_POSIX_C_SOURCE=200809L", "-fPIC", "-shared",
           "-pthread", "-o", tmp, _SRC, _SRC_MOVE, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    newest = max(os.path.getmtime(_SRC), os.path.getmtime(_SRC_MOVE))
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < newest:
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f64.restype = ctypes.c_double
    lib.oracle_gemm_i8i64.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, ctypes.c_int]
    lib.oracle_gemm_i8i64.restype = ctypes.c_int
    lib.oracle_gemm_f16f64.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, vp, ctypes.c_int]
    lib.oracle_gemm_f16f64.restype = ctypes.c_int
    lib.oracle_gemm_i8i64_at.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, vp, i64, vp]
    lib.oracle_gemm_i8i64_at.restype = ctypes.c_int
    lib.oracle_gemm_f16f64_at.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, vp, i64, vp, vp]
    lib.oracle_gemm_f16f64_at.restype = ctypes.c_int
    lib.oracle_gemm_f32f64.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, vp, ctypes.c_int]
    lib.oracle_gemm_f32f64.restype = ctypes.c_int
    lib.oracle_gemm_f32f64_at.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, vp, i64, vp, vp]
    lib.oracle_gemm_f32f64_at.restype = ctypes.c_int
    for name in ("oracle_copy_u32", "oracle_transpose_u32"):
        getattr(lib, name).argtypes = [i64, i64, vp, i64, vp, i64]
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def host_threads() -> int:
    """Threads this process may run on (the CPU set it is pinned to)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _operand(x: np.ndarray, dtype) -> tuple[int, int, int, int]:
    """(rows, cols, pointer, leading dimension) of a row-major 2-D operand.

    Rows may be strided (a view into a wider matrix); elements within a row
    must be contiguous."""
    if x.dtype != dtype or x.ndim != 2:
        raise TypeError("expected a 2-D %s array, got %s %s" % (np.dtype(dtype), x.dtype, x.shape))
    item = x.itemsize
    if x.size == 0:
        return x.shape[0], x.shape[1], x.ctypes.data, max(1, x.shape[1])
    if x.shape[1] > 1 and x.strides[1] != item:
        raise ValueError("elements within a row must be contiguous")
    ld = x.strides[0] // item if x.shape[0] > 1 else max(1, x.shape[1])
    if x.shape[0] > 1 and x.strides[0] % item:
        raise ValueError("row stride must be a whole number of elements")
    return x.shape[0], x.shape[1], x.ctypes.data, max(ld, 1)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError("%s failed with status %d" % (what, rc))


def gemm_i8(A: np.ndarray, B: np.ndarray, threads: int | None = None) -> np.ndarray:
    """C = A.B for int8 A (M x K) and B (K x N); returns int64 C (M x N)."""
    M, K, pa, lda = _operand(A, np.int8)
    K2, N, pb, ldb = _operand(B, np.int8)
    if K != K2:
        raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))
    C = np.empty((M, N), dtype=np.int64)
    _check(_load().oracle_gemm_i8i64(M, N, K, pa, lda, pb, ldb, C.ctypes.data,
                                     threads or host_threads()), "oracle_gemm_i8i64")
    return C


def gemm_f16(A: np.ndarray, B: np.ndarray, threads: int | None = None,
             with_scale: bool = True):
    """C = A.B for binary16 A (M x K) and B (K x N), given as float16 or uint16
    bit arrays; returns (C, S) as float64 arrays, S = sum_k |a_ik b_kj|
    (None when with_scale is False)."""
    A = A.view(np.uint16) if A.dtype == np.float16 else A
    B = B.view(np.uint16) if B.dtype == np.float16 else B
    M, K, pa, lda = _operand(A, np.uint16)
    K2, N, pb, ldb = _operand(B, np.uint16)
    if K != K2:
        raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))
    C = np.empty((M, N), dtype=np.float64)
    S = np.empty((M, N), dtype=np.float64) if with_scale else None
    _check(_load().oracle_gemm_f16f64(M, N, K, pa, lda, pb, ldb, C.ctypes.data,
                                      S.ctypes.data if S is not None else None,
                                      threads or host_threads()), "oracle_gemm_f16f64")
    return C, S


def gemm_f32(A: np.ndarray, B: np.ndarray, threads: int | None = None,
             with_scale: bool = True):
    """C = A.B for binary32 A (M x K) and B (K x N); returns (C, S) as float64
    arrays, S = sum_k |a_ik b_kj| (None when with_scale is False)."""
    M, K, pa, lda = _operand(A, np.float32)
    K2, N, pb, ldb = _operand(B, np.float32)
    if K != K2:
        raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))
    C = np.empty((M, N), dtype=np.float64)
    S = np.empty((M, N), dtype=np.float64) if with_scale else None
    _check(_load().oracle_gemm_f32f64(M, N, K, pa, lda, pb, ldb, C.ctypes.data,
                                      S.ctypes.data if S is not None else None,
                                      threads or host_threads()), "oracle_gemm_f32f64")
    return C, S


def _index_arrays(rows, cols):
    r = np.ascontiguousarray(rows, dtype=np.int64)
    c = np.ascontiguousarray(cols, dtype=np.int64)
    if r.shape != c.shape or r.ndim != 1:
        raise ValueError("rows and cols must be 1-D and of equal length")
    return r, c


def gemm_i8_at(A: np.ndarray, B: np.ndarray, rows, cols) -> np.ndarray:
    """The elements C[rows[t], cols[t]] of C = A.B (int8 inputs), as int64."""
    M, K, pa, lda = _operand(A, np.int8)
    K2, N, pb, ldb = _operand(B, np.int8)
    if K != K2:
        raise ValueError("inner dimensions differ")
    r, c = _index_arrays(rows, cols)
    out = np.empty(r.shape, dtype=np.int64)
    _check(_load().oracle_gemm_i8i64_at(M, N, K, pa, lda, pb, ldb, r.ctypes.data,
                                        c.ctypes.data, r.size, out.ctypes.data),
           "oracle_gemm_i8i64_at")
    return out


def gemm_f16_at(A: np.ndarray, B: np.ndarray, rows, cols):
    """The elements (C, S)[rows[t], cols[t]] of C = A.B (binary16 inputs)."""
    A = A.view(np.uint16) if A.dtype == np.float16 else A
    B = B.view(np.uint16) if B.dtype == np.float16 else B
    M, K, pa, lda = _operand(A, np.uint16)
    K2, N, pb, ldb = _operand(B, np.uint16)
    if K != K2:
        raise ValueError("inner dimensions differ")
    r, c = _index_arrays(rows, cols)
    out = np.empty(r.shape, dtype=np.float64)
    out_s = np.empty(r.shape, dtype=np.float64)
    _check(_load().oracle_gemm_f16f64_at(M, N, K, pa, lda, pb, ldb, r.ctypes.data,
                                         c.ctypes.data, r.size, out.ctypes.data,
                                         out_s.ctypes.data), "oracle_gemm_f16f64_at")
    return out, out_s


def gemm_f32_at(A: np.ndarray, B: np.ndarray, rows, cols):
    """The elements (C, S)[rows[t], cols[t]] of C = A.B (binary32 inputs)."""
    M, K, pa, lda = _operand(A, np.float32)
    K2, N, pb, ldb = _operand(B, np.float32)
    if K != K2:
        raise ValueError("inner dimensions differ")
    r, c = _index_arrays(rows, cols)
    out = np.empty(r.shape, dtype=np.float64)
    out_s = np.empty(r.shape, dtype=np.float64)
    _check(_load().oracle_gemm_f32f64_at(M, N, K, pa, lda, pb, ldb, r.ctypes.data,
                                         c.ctypes.data, r.size, out.ctypes.data,
                                         out_s.ctypes.data), "oracle_gemm_f32f64_at")
    return out, out_s


def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    """The oracle's own binary16 widening, element by element."""
    lib = _load()
    flat = np.ascontiguousarray(bits, dtype=np.uint16).ravel()
    return np.array([lib.oracle_f16_to_f64(int(h)) for h in flat], dtype=np.float64).reshape(
        np.shape(bits))


def _u32_operand(x: np.ndarray):
    """A 2-D array of 32-bit elements (float32 or uint32) as uint32 bits."""
    if x.dtype == np.float32:
        x = x.view(np.uint32)
    return _operand(x, np.uint32)


def copy_u32(x: np.ndarray) -> np.ndarray:
    """out[i][j] = x[i][j] for a 2-D array of 32-bit elements (returns uint32
    bits; "fixing GPU kernels by hand", the copy that bounds the transpose)."""
    rows, cols, px, ldx = _u32_operand(x)
    out = np.empty((rows, cols), dtype=np.uint32)
    _check(_load().oracle_copy_u32(rows, cols, px, ldx, out.ctypes.data, max(1, cols)),
           "oracle_copy_u32")
    return out


def transpose_u32(x: np.ndarray) -> np.ndarray:
    """out[j][i] = x[i][j] for a 2-D array of 32-bit elements (returns uint32
    bits; "fixing GPU kernels by hand", the transpose exercise)."""
    rows, cols, px, ldx = _u32_operand(x)
    out = np.empty((cols, rows), dtype=np.uint32)
    _check(_load().oracle_transpose_u32(rows, cols, px, ldx, out.ctypes.data, max(1, rows)),
           "oracle_transpose_u32")
    return out
