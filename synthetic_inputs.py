"""Seeded synthetic operands for the tiled dense GEMM, shared by the tests,
the benchmark and the smoke check.

This module only draws numbers; it holds no step of the product.  Every array
is host memory (numpy), drawn from numpy's PCG64 generator
(``numpy.random.default_rng(seed)``), so a seed names the same bytes on every
machine:

* binary16 operands are a float32 draw rounded to the nearest binary16
  (numpy's ``astype(np.float16)``, round-to-nearest-even), returned as the
  raw uint16 bit patterns the GPU library takes;
* int8 operands are uniform integers on [-128, 127] inclusive;
* binary32 operands are the float32 draws themselves.

The pages measure a 4096 x 4096 x 4096 integer GEMM ("Pipeline GPU Kernel",
Step 2 and Step 6) and name no dataset; the five workloads below are that
shape and its neighbours, drawn synthetically.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def f16_normal(rows: int, cols: int, seed: int) -> np.ndarray:
    """N(0, 1) draws rounded to binary16; returns uint16 bits, shape (rows, cols)."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((rows, cols), dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_uniform(rows: int, cols: int, seed: int, lo: float = -1.0, hi: float = 1.0) -> np.ndarray:
    """Uniform [lo, hi) draws rounded to binary16; returns uint16 bits."""
    rng = np.random.default_rng(seed)
    x = rng.random((rows, cols), dtype=np.float32) * np.float32(hi - lo) + np.float32(lo)
    return x.astype(np.float16).view(np.uint16)


def f16_integers(rows: int, cols: int, seed: int, lo: int = -8, hi: int = 8) -> np.ndarray:
    """Integers uniform on [lo, hi] inclusive, stored as binary16 bits (exact)."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=(rows, cols)).astype(np.float16).view(np.uint16)


def f16_subnormals(rows: int, cols: int, seed: int) -> np.ndarray:
    """binary16 subnormals: random sign, exponent field 0, mantissa field
    uniform on [1, 1023], i.e. values m * 2^-24; returns uint16 bits."""
    rng = np.random.default_rng(seed)
    sign = rng.integers(0, 2, size=(rows, cols), dtype=np.uint16) << np.uint16(15)
    mant = rng.integers(1, 1024, size=(rows, cols), dtype=np.uint16)
    return sign | mant


def f32_normal(rows: int, cols: int, seed: int) -> np.ndarray:
    """N(0, 1) float32 draws, shape (rows, cols)."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((rows, cols), dtype=np.float32)


def f32_integers(rows: int, cols: int, seed: int, lo: int = -8, hi: int = 8) -> np.ndarray:
    """Integers uniform on [lo, hi] inclusive, as float32 (exact)."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=(rows, cols)).astype(np.float32)


def i8_uniform(rows: int, cols: int, seed: int) -> np.ndarray:
    """int8 uniform on [-128, 127] inclusive."""
    rng = np.random.default_rng(seed)
    return rng.integers(-128, 128, size=(rows, cols), dtype=np.int8)


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "i8" (INT8 in, INT32 out), "f16" (FP16 in, FP32 out), "f32"
    M: int
    N: int
    K: int
    dist: str           # "uniform_i8", "normal", "uniform_pm1"
    seed_a: int
    seed_b: int

    def operands(self):
        """(A, B) host arrays: A is M x K, B is K x N, row-major."""
        if self.dist == "uniform_i8":
            return i8_uniform(self.M, self.K, self.seed_a), i8_uniform(self.K, self.N, self.seed_b)
        if self.dist == "normal" and self.dtype == "f32":
            return f32_normal(self.M, self.K, self.seed_a), f32_normal(self.K, self.N, self.seed_b)
        if self.dist == "normal":
            return f16_normal(self.M, self.K, self.seed_a), f16_normal(self.K, self.N, self.seed_b)
        if self.dist == "uniform_pm1":
            return (f16_uniform(self.M, self.K, self.seed_a),
                    f16_uniform(self.K, self.N, self.seed_b))
        raise ValueError(self.dist)


def _wl(idx: int, name: str, dtype: str, M: int, N: int, K: int, dist: str) -> Workload:
    # workload c draws A from seed 1000*c + 1 and B from seed 1000*c + 2
    return Workload(name, dtype, M, N, K, dist, 1000 * idx + 1, 1000 * idx + 2)


WORKLOADS = {
    "int8_256": _wl(1, "int8_256", "i8", 256, 256, 256, "uniform_i8"),
    "fp16_1024": _wl(2, "fp16_1024", "f16", 1024, 1024, 1024, "normal"),
    "int8_4096": _wl(3, "int8_4096", "i8", 4096, 4096, 4096, "uniform_i8"),
    "fp16_4096": _wl(4, "fp16_4096", "f16", 4096, 4096, 4096, "normal"),
    "fp16_skinny": _wl(5, "fp16_skinny", "f16", 16384, 64, 8192, "uniform_pm1"),
    # a ragged neighbour of the 4096^3 workload: no dimension a tile multiple,
    # N and K whole 16-byte chunks (the bounds-checked direct-to-LDS loop)
    "fp16_ragged": _wl(6, "fp16_ragged", "f16", 4000, 4000, 4000, "normal"),
    # the pages' third data type (FP32 in, FP32 accumulate) at the headline shape
    "fp32_4096": _wl(7, "fp32_4096", "f32", 4096, 4096, 4096, "normal"),
    # one GPU's share when the 4096^3 products are split by C row panels over
    # 8 GPUs: the same seeds, so A is exactly the first 512 rows of the full
    # workload's A (the generator fills row-major) and B is all of it
    "fp16_shard8": _wl(4, "fp16_shard8", "f16", 512, 4096, 4096, "normal"),
    "int8_shard8": _wl(3, "int8_shard8", "i8", 512, 4096, 4096, "uniform_i8"),
}
