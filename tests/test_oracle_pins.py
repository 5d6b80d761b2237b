"""Pins for the CPU oracle: each checks it against something other than itself.

The pages print no GEMM values, so the pins are exact arithmetic (Python
integers, exact fractions), closed forms (identity, rank-1, the exhaustive
int8 product table), invariants (K-split additivity, the transpose identity)
and library routines (numpy's matmul in int64/float64 and numpy's binary16
widening).  Each is chosen so that a plausible slip in the oracle -- a dropped
k term, a wrong index or leading dimension, a transposed operand, a wrong
exponent bias in the binary16 decode -- fails at least one of them; the last
tests plant such slips on the CPU and show that the pins catch them.
"""
from fractions import Fraction
import itertools

import numpy as np
import pytest

import oracle
import synthetic_inputs as si

EPS64 = 2.0 ** -53


def _exact_f16(bits):
    """Exact rational value of each binary16 bit pattern (via float, which
    holds every binary16 value exactly)."""
    return [[Fraction(float(v)) for v in row] for row in bits.view(np.float16).astype(np.float64)]


# --- binary16 widening --------------------------------------------------------

def test_f16_widening_matches_numpy_for_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros and infinities keep their sign
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_f16_widening_known_values():
    # values fixed by the binary16 format itself
    known = {0x3C00: 1.0, 0xC000: -2.0, 0x7BFF: 65504.0, 0x0001: 2.0 ** -24,
             0x0400: 2.0 ** -14, 0x3555: 1365.0 / 4096.0, 0x8000: -0.0}
    got = oracle.f16_to_f64(np.array(list(known), dtype=np.uint16))
    assert list(got) == list(known.values())


# --- brute force on tiny inputs -------------------------------------------------

TINY = list(itertools.product(range(1, 5), repeat=3)) + [(9, 7, 5), (5, 9, 7), (7, 5, 9), (8, 8, 8)]


@pytest.mark.parametrize("M,N,K", TINY)
def test_brute_force_int8(M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    A = rng.integers(-128, 128, size=(M, K), dtype=np.int8)
    B = rng.integers(-128, 128, size=(K, N), dtype=np.int8)
    C = oracle.gemm_i8(A, B, threads=3)
    for i in range(M):
        for j in range(N):
            assert int(C[i, j]) == sum(int(A[i, k]) * int(B[k, j]) for k in range(K))


@pytest.mark.parametrize("M,N,K", TINY)
def test_brute_force_f16_exact_fractions(M, N, K):
    A = si.f16_normal(M, K, seed=M * 100 + N * 10 + K)
    B = si.f16_normal(K, N, seed=M * 100 + N * 10 + K + 7)
    C, S = oracle.gemm_f16(A, B, threads=2)
    Ae, Be = _exact_f16(A), _exact_f16(B)
    for i in range(M):
        for j in range(N):
            prods = [Ae[i][k] * Be[k][j] for k in range(K)]
            exact = sum(prods, Fraction(0))
            scale = sum((abs(p) for p in prods), Fraction(0))
            bound = K * EPS64 * float(scale)
            assert abs(Fraction(C[i, j]) - exact) <= Fraction(bound)
            assert abs(Fraction(S[i, j]) - scale) <= Fraction(bound)


# --- exhaustive int8 product table ------------------------------------------------

def test_subnormal_products_closed_form():
    """Subnormal A (m * 2^-24, from its bit fields alone) times integer B:
    C = (sum_k s_ik m_ik b_kj) * 2^-24 exactly, computed in int64 from the
    sign and mantissa fields, with no binary16 decode at all."""
    M, N, K = 37, 29, 300
    A = si.f16_subnormals(M, K, seed=5)
    B = si.f16_integers(K, N, seed=6)
    sign = np.where(A >> 15, -1, 1).astype(np.int64)
    m = (A & 0x3FF).astype(np.int64) * sign
    b = B.view(np.float16).astype(np.int64)
    want = (m @ b).astype(np.float64) * 2.0 ** -24
    got, S = oracle.gemm_f16(A, B)
    assert np.array_equal(got, want)
    assert np.array_equal(S, (np.abs(m) @ np.abs(b)).astype(np.float64) * 2.0 ** -24)


def test_exhaustive_int8_product_table():
    vals = np.arange(-128, 128, dtype=np.int16).astype(np.int8)
    A = vals.reshape(256, 1).copy()
    B = vals[::-1].reshape(1, 256).copy()
    C = oracle.gemm_i8(A, B)
    a = [int(v) for v in vals]
    b = [int(v) for v in vals[::-1]]
    for i in range(256):
        assert [int(x) for x in C[i]] == [a[i] * bj for bj in b]
    assert C.min() == -128 * 127 and C.max() == 16384


# --- identity --------------------------------------------------------------------

def test_identity_int8():
    A = si.i8_uniform(37, 53, seed=1)
    I53 = np.eye(53, dtype=np.int8)
    I37 = np.eye(37, dtype=np.int8)
    assert np.array_equal(oracle.gemm_i8(A, I53), A.astype(np.int64))
    assert np.array_equal(oracle.gemm_i8(I37, A), A.astype(np.int64))


def test_identity_f16():
    A = si.f16_normal(29, 41, seed=2)
    one = np.float16(1.0).view(np.uint16)
    I41 = np.where(np.eye(41, dtype=bool), one, np.uint16(0)).astype(np.uint16)
    I29 = np.where(np.eye(29, dtype=bool), one, np.uint16(0)).astype(np.uint16)
    Af = A.view(np.float16).astype(np.float64)
    assert np.array_equal(oracle.gemm_f16(A, I41)[0], Af)
    assert np.array_equal(oracle.gemm_f16(I29, A)[0], Af)


# --- all-ones and rank-1 closed forms ---------------------------------------------

def test_all_ones_int8():
    M, N, K = 33, 47, 300
    B = si.i8_uniform(K, N, seed=3)
    A = si.i8_uniform(M, K, seed=4)
    ones_a = np.ones((M, K), dtype=np.int8)
    ones_b = np.ones((K, N), dtype=np.int8)
    colsum = [sum(int(B[k, j]) for k in range(K)) for j in range(N)]
    rowsum = [sum(int(A[i, k]) for k in range(K)) for i in range(M)]
    C1 = oracle.gemm_i8(ones_a, B)
    C2 = oracle.gemm_i8(A, ones_b)
    for i in range(M):
        assert [int(x) for x in C1[i]] == colsum
        assert [int(x) for x in C2[i]] == [rowsum[i]] * N


def test_rank1_int8_extremes():
    # A[i][k] = u_i, B[k][j] = v_j  ->  C_ij = K * u_i * v_j (= rowsum_i * colsum_j / K)
    M, N, K = 16, 16, 4096
    u = np.array([-128, 127, 1, -1, 0, 64, -64, 5] * 2, dtype=np.int8)
    v = np.array([127, -128, -1, 1, 3, 0, 100, -7] * 2, dtype=np.int8)
    A = np.repeat(u.reshape(M, 1), K, axis=1)
    B = np.repeat(v.reshape(1, N), K, axis=0)
    C = oracle.gemm_i8(A, B)
    for i in range(M):
        for j in range(N):
            assert int(C[i, j]) == K * int(u[i]) * int(v[j])
    assert int(C.max()) == 4096 * 16384


def test_rank1_f16():
    M, N, K = 8, 9, 1000
    u = si.f16_integers(M, 1, seed=5)
    v = si.f16_integers(1, N, seed=6)
    A = np.repeat(u, K, axis=1)
    B = np.repeat(v, K, axis=0)
    C, S = oracle.gemm_f16(A, B)
    uf = u.view(np.float16).astype(np.float64)[:, 0]
    vf = v.view(np.float16).astype(np.float64)[0]
    for i in range(M):
        for j in range(N):
            assert C[i, j] == K * uf[i] * vf[j]
            assert S[i, j] == K * abs(uf[i] * vf[j])


# --- K-split additivity (also exercises leading dimensions) -------------------------

@pytest.mark.parametrize("k1", [1, 17, 64, 99])
def test_k_split_additivity_int8(k1):
    M, N, K = 23, 31, 100
    A = si.i8_uniform(M, K, seed=7)
    B = si.i8_uniform(K, N, seed=8)
    full = oracle.gemm_i8(A, B)
    part = oracle.gemm_i8(A[:, :k1], B[:k1, :]) + oracle.gemm_i8(A[:, k1:], B[k1:, :])
    assert np.array_equal(full, part)


@pytest.mark.parametrize("k1", [1, 50, 99])
def test_k_split_additivity_f16_integer_valued(k1):
    M, N, K = 19, 21, 100
    A = si.f16_integers(M, K, seed=9)
    B = si.f16_integers(K, N, seed=10)
    full = oracle.gemm_f16(A, B)[0]
    part = oracle.gemm_f16(A[:, :k1], B[:k1, :])[0] + oracle.gemm_f16(A[:, k1:], B[k1:, :])[0]
    assert np.array_equal(full, part)


def test_leading_dimensions_match_contiguous_copies():
    big_a = si.i8_uniform(40, 70, seed=11)
    big_b = si.i8_uniform(60, 90, seed=12)
    A, B = big_a[3:35, 5:50], big_b[2:47, 7:80]
    assert np.array_equal(oracle.gemm_i8(A, B), oracle.gemm_i8(A.copy(), B.copy()))
    fa = si.f16_normal(40, 70, seed=13)[3:35, 5:50]
    fb = si.f16_normal(60, 90, seed=14)[2:47, 7:80]
    C1, S1 = oracle.gemm_f16(fa, fb)
    C2, S2 = oracle.gemm_f16(fa.copy(), fb.copy())
    assert np.array_equal(C1, C2) and np.array_equal(S1, S2)


# --- numpy matmul in int64 / float64 --------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(64, 64, 64), (256, 128, 512), (100, 300, 257)])
def test_numpy_matmul_int8(M, N, K):
    A = si.i8_uniform(M, K, seed=M + N)
    B = si.i8_uniform(K, N, seed=M + K)
    assert np.array_equal(oracle.gemm_i8(A, B), A.astype(np.int64) @ B.astype(np.int64))


@pytest.mark.parametrize("M,N,K", [(64, 64, 64), (256, 128, 512), (100, 300, 257)])
def test_numpy_matmul_f16(M, N, K):
    A = si.f16_normal(M, K, seed=M + N)
    B = si.f16_normal(K, N, seed=M + K)
    Af = A.view(np.float16).astype(np.float64)
    Bf = B.view(np.float16).astype(np.float64)
    C, S = oracle.gemm_f16(A, B)
    ref = Af @ Bf
    ref_s = np.abs(Af) @ np.abs(Bf)
    # products are exact in double; the two sums differ only by rounding order
    assert np.all(np.abs(C - ref) <= 2 * K * EPS64 * ref_s)
    assert np.all(np.abs(S - ref_s) <= 2 * K * EPS64 * ref_s)


# --- transpose identity ----------------------------------------------------------------

def test_transpose_identity():
    A = si.i8_uniform(45, 67, seed=15)
    B = si.i8_uniform(67, 38, seed=16)
    assert np.array_equal(oracle.gemm_i8(B.T.copy(), A.T.copy()), oracle.gemm_i8(A, B).T)
    fa = si.f16_normal(45, 67, seed=17)
    fb = si.f16_normal(67, 38, seed=18)
    assert np.array_equal(oracle.gemm_f16(fb.T.copy(), fa.T.copy())[0], oracle.gemm_f16(fa, fb)[0].T)


# --- degenerate shapes and thread count ----------------------------------------------------

def test_k_zero_gives_zeros_and_empty_shapes():
    A = np.zeros((5, 0), dtype=np.int8)
    B = np.zeros((0, 7), dtype=np.int8)
    assert np.array_equal(oracle.gemm_i8(A, B), np.zeros((5, 7), dtype=np.int64))
    assert oracle.gemm_i8(np.zeros((0, 4), np.int8), np.zeros((4, 3), np.int8)).shape == (0, 3)
    C, S = oracle.gemm_f16(np.zeros((3, 0), np.uint16), np.zeros((0, 2), np.uint16))
    assert np.array_equal(C, np.zeros((3, 2))) and np.array_equal(S, np.zeros((3, 2)))


def test_thread_count_does_not_change_results():
    A = si.f16_normal(61, 77, seed=19)
    B = si.f16_normal(77, 83, seed=20)
    C1, S1 = oracle.gemm_f16(A, B, threads=1)
    C7, S7 = oracle.gemm_f16(A, B, threads=7)
    assert np.array_equal(C1, C7) and np.array_equal(S1, S7)


# --- single-element form agrees with the full product ------------------------------------

def test_elementwise_form_matches_full_product():
    A = si.i8_uniform(70, 90, seed=21)
    B = si.i8_uniform(90, 50, seed=22)
    rows = np.array([0, 69, 13, 42, 7])
    cols = np.array([0, 49, 25, 1, 33])
    assert np.array_equal(oracle.gemm_i8_at(A, B, rows, cols), oracle.gemm_i8(A, B)[rows, cols])
    fa = si.f16_normal(70, 90, seed=23)
    fb = si.f16_normal(90, 50, seed=24)
    C, S = oracle.gemm_f16(fa, fb)
    c, s = oracle.gemm_f16_at(fa, fb, rows, cols)
    assert np.array_equal(c, C[rows, cols]) and np.array_equal(s, S[rows, cols])


def test_elementwise_form_on_strided_views():
    """The single-element forms read A and B through their leading
    dimensions: on views into wider matrices whose padding holds other
    values, every requested element equals numpy's product of the views
    (int64 exactly; float64 within rounding of the summation order) and the
    full routine's element bit for bit.  Taking N for ldb or K for lda would
    read the padding and fail."""
    rng = np.random.default_rng(31)
    M, N, K = 37, 29, 53
    Aw = si.i8_uniform(M, K + 11, seed=32)
    Bw = si.i8_uniform(K, N + 7, seed=33)
    A, B = Aw[:, 3:3 + K], Bw[:, 5:5 + N]
    assert A.strides[0] == K + 11 and B.strides[0] == N + 7
    rows = rng.integers(0, M, 200)
    cols = rng.integers(0, N, 200)
    ref = (A.astype(np.int64) @ B.astype(np.int64))[rows, cols]
    assert np.array_equal(oracle.gemm_i8_at(A, B, rows, cols), ref)
    assert np.array_equal(oracle.gemm_i8(A, B)[rows, cols], ref)
    for wide, widen, full, at in (
            (lambda r, c, s: si.f16_normal(r, c, s), lambda x: x.view(np.float16).astype(np.float64),
             oracle.gemm_f16, oracle.gemm_f16_at),
            (lambda r, c, s: si.f32_normal(r, c, s), lambda x: x.astype(np.float64),
             oracle.gemm_f32, oracle.gemm_f32_at)):
        Aw, Bw = wide(M, K + 11, 34), wide(K, N + 7, 35)
        A, B = Aw[:, 3:3 + K], Bw[:, 5:5 + N]
        c, s = at(A, B, rows, cols)
        C, S = full(A, B)
        assert np.array_equal(c, C[rows, cols]) and np.array_equal(s, S[rows, cols])
        ref = (widen(A) @ widen(B))[rows, cols]
        ref_s = (np.abs(widen(A)) @ np.abs(widen(B)))[rows, cols]
        assert np.all(np.abs(c - ref) <= 1e-12 * ref_s)
        assert np.allclose(s, ref_s, rtol=1e-12, atol=0.0)


def test_elementwise_form_rank1_closed_form_at_full_size():
    # 4096-long sums at the largest magnitudes int8 allows
    K = 4096
    A = np.full((4, K), -128, dtype=np.int8)
    B = np.full((K, 3), -128, dtype=np.int8)
    out = oracle.gemm_i8_at(A, B, [0, 3, 2], [0, 2, 1])
    assert list(out) == [K * 16384] * 3


# --- planted mistakes are caught -----------------------------------------------------------

def test_pins_catch_a_dropped_last_k_slice():
    """Dropping the last BK-wide slice of K (the forgotten-epilogue bug of
    "Pipeline GPU Kernel", Common Pitfalls) is visible to the all-ones pin:
    the sum over K-BK terms is K-BK, not K."""
    K, BK = 256, 64
    ones_a = np.ones((4, K), dtype=np.int8)
    ones_b = np.ones((K, 4), dtype=np.int8)
    planted = oracle.gemm_i8(ones_a[:, :K - BK], ones_b[:K - BK, :])
    assert np.all(planted == K - BK)
    assert not np.all(planted == K)
    assert np.all(oracle.gemm_i8(ones_a, ones_b) == K)


def test_pins_catch_a_transposed_operand():
    A = si.i8_uniform(8, 8, seed=25)
    B = si.i8_uniform(8, 8, seed=26)
    good = oracle.gemm_i8(A, B)
    planted = oracle.gemm_i8(A, B.T.copy())
    assert not np.array_equal(planted, A.astype(np.int64) @ B.astype(np.int64))
    assert np.array_equal(good, A.astype(np.int64) @ B.astype(np.int64))
