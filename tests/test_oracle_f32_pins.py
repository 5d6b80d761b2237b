"""Pins for the FP32-input oracle ("Pipeline GPU Kernel", Step 5: FP32 scalar
FFMA is the third data type), each against something other than itself:
exact rational arithmetic on tiny shapes, numpy's float64 matmul, closed forms
(identity, all-ones, rank-1, the scale S), K-split additivity and the
transpose identity.  The last tests plant plausible slips on the CPU (a
dropped last k, operands narrowed to binary16) and show the pins catch them."""
from fractions import Fraction
import itertools

import numpy as np
import pytest

import oracle
import synthetic_inputs as si

EPS64 = 2.0 ** -53
TINY = [s for s in itertools.product(range(1, 5), repeat=3)] + [(7, 5, 9), (9, 9, 9)]


def _exact(x):
    return [[Fraction(float(v)) for v in row] for row in x.astype(np.float64)]


@pytest.mark.parametrize("M,N,K", TINY)
def test_brute_force_exact_fractions(M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    A = (rng.standard_normal((M, K)) * 3).astype(np.float32)
    B = (rng.standard_normal((K, N)) * 3).astype(np.float32)
    C, S = oracle.gemm_f32(A, B)
    ea, eb = _exact(A), _exact(B)
    for i in range(M):
        for j in range(N):
            exact = sum(ea[i][k] * eb[k][j] for k in range(K))
            scale = sum(abs(ea[i][k] * eb[k][j]) for k in range(K))
            assert abs(Fraction(C[i, j]) - exact) <= K * EPS64 * scale
            assert abs(Fraction(S[i, j]) - scale) <= K * EPS64 * scale


@pytest.mark.parametrize("M,N,K", [(64, 64, 64), (200, 130, 257)])
def test_numpy_float64_matmul(M, N, K):
    A, B = si.f32_normal(M, K, 1), si.f32_normal(K, N, 2)
    C, S = oracle.gemm_f32(A, B)
    ref = A.astype(np.float64) @ B.astype(np.float64)
    assert np.all(np.abs(C - ref) <= 2 * K * EPS64 * S)
    assert np.allclose(S, np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64)), rtol=1e-12)


def test_identity_is_exact():
    A = si.f32_normal(50, 40, 3)
    C, _ = oracle.gemm_f32(A, np.eye(40, dtype=np.float32))
    assert np.array_equal(C, A.astype(np.float64))
    C, _ = oracle.gemm_f32(np.eye(50, dtype=np.float32), A)
    assert np.array_equal(C, A.astype(np.float64))


def test_all_ones_and_rank1_closed_forms():
    M, N, K = 33, 17, 300
    C, S = oracle.gemm_f32(np.ones((M, K), np.float32), np.ones((K, N), np.float32))
    assert np.all(C == K) and np.all(S == K)
    u = np.arange(-16, 17, dtype=np.float32)[:M].reshape(M, 1)
    v = np.arange(N, dtype=np.float32).reshape(1, N) - 8
    A = np.repeat(u, K, axis=1)
    B = np.repeat(v, K, axis=0)
    C, S = oracle.gemm_f32(A, B)
    assert np.array_equal(C, K * (u.astype(np.float64) @ v.astype(np.float64)))
    assert np.array_equal(S, K * np.abs(u.astype(np.float64) @ v.astype(np.float64)))


@pytest.mark.parametrize("k1", [1, 50, 99])
def test_k_split_additivity_integer_valued(k1):
    A, B = si.f32_integers(40, 100, 5), si.f32_integers(100, 30, 6)
    C, _ = oracle.gemm_f32(A, B)
    C1, _ = oracle.gemm_f32(A[:, :k1], B[:k1, :])
    C2, _ = oracle.gemm_f32(A[:, k1:], B[k1:, :])
    assert np.array_equal(C, C1 + C2)


def test_transpose_identity():
    A, B = si.f32_integers(30, 45, 7), si.f32_integers(45, 20, 8)
    C, _ = oracle.gemm_f32(A, B)
    Ct, _ = oracle.gemm_f32(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T))
    assert np.array_equal(C, Ct.T)


def test_elementwise_form_matches_full_product():
    A, B = si.f32_normal(70, 90, 9), si.f32_normal(90, 60, 10)
    C, S = oracle.gemm_f32(A, B)
    rows = np.array([0, 69, 33, 5]); cols = np.array([0, 59, 17, 44])
    c, s = oracle.gemm_f32_at(A, B, rows, cols)
    assert np.array_equal(c, C[rows, cols]) and np.array_equal(s, S[rows, cols])


def test_pins_catch_a_dropped_last_k():
    """An oracle that stops one k early (same leading dimensions) fails the
    all-ones closed form and the numpy pin."""
    M, N, K = 8, 8, 64
    A, B = si.f32_normal(M, K, 11), si.f32_normal(K, N, 12)
    short, _ = oracle.gemm_f32(A[:, :K - 1], B[:K - 1, :])
    ref = A.astype(np.float64) @ B.astype(np.float64)
    _, S = oracle.gemm_f32(A, B)
    assert not np.all(np.abs(short - ref) <= 2 * K * EPS64 * S)
    ones, _ = oracle.gemm_f32(np.ones((M, K - 1), np.float32), np.ones((K - 1, N), np.float32))
    assert not np.all(ones == K)


def test_pins_catch_narrowed_operands():
    """An oracle that rounds its binary32 inputs to binary16 first fails the
    exact-fraction pin on values binary16 cannot hold."""
    A = np.array([[1.0 + 2.0 ** -20, 3.0]], dtype=np.float32)
    B = np.array([[1.0], [2.0 ** -20]], dtype=np.float32)
    narrowed, _ = oracle.gemm_f32(A.astype(np.float16).astype(np.float32),
                                  B.astype(np.float16).astype(np.float32))
    exact = Fraction(float(A[0, 0])) * 1 + 3 * Fraction(float(B[1, 0]))
    good, _ = oracle.gemm_f32(A, B)
    assert Fraction(good[0, 0]) == exact
    assert Fraction(narrowed[0, 0]) != exact
