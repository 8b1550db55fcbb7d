"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test fixes the oracle to something independent: exact integer
arithmetic in Python, closed forms (identity, all-ones), the pages' 8x8 / T=4
block decomposition, an fp64 BLAS witness and the classical error bound.  A
dropped term, a wrong sign or index, a transposed operand or a silent drop to
fp32 accumulation each fails at least one of them (see the planted-mistake
tests at the bottom, which plant such mistakes in copies of the oracle's
output or inputs, never in the oracle itself).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from gemm_inputs import make, make_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")


def _exact_int_product(a: np.ndarray, b: np.ndarray) -> list[list[int]]:
    """Brute force in Python integers: no rounding anywhere."""
    ai = [[int(v) for v in row] for row in a]
    bi = [[int(v) for v in row] for row in b]
    M, K = a.shape
    N = b.shape[1]
    return [[sum(ai[i][k] * bi[k][j] for k in range(K)) for j in range(N)] for i in range(M)]


# P1: brute force against exact integer sums on every tiny shape.
def test_brute_force_tiny_shapes_exact():
    dims = (0, 1, 2, 3, 5, 8)
    rng = np.random.default_rng(1234)
    for M, N, K in itertools.product(dims, dims, dims):
        a = rng.integers(-9, 10, (M, K)).astype(np.float32)
        b = rng.integers(-9, 10, (K, N)).astype(np.float32)
        c = oracle.gemm(a, b)
        assert c.shape == (M, N)
        exact = _exact_int_product(a, b)
        for i in range(M):
            for j in range(N):
                assert c[i, j] == exact[i][j], (M, N, K, i, j)


def test_literal_triple_loop_bit_identical():
    """The oracle equals the literal i-j-k loop in fp64 followed by one fp32 rounding."""
    rng = np.random.default_rng(7)
    for M, N, K in [(3, 4, 5), (7, 1, 13), (1, 9, 33), (6, 6, 64)]:
        a = rng.standard_normal((M, K), dtype=np.float32)
        b = rng.standard_normal((K, N), dtype=np.float32)
        c = oracle.gemm(a, b)
        for i in range(M):
            for j in range(N):
                s = 0.0
                for k in range(K):
                    s += float(a[i, k]) * float(b[k, j])
                assert c[i, j] == np.float32(s), (M, N, K, i, j)


def test_nonsquare_orientation():
    """A (2x3) x B (3x4) with distinct entries: catches a transposed operand."""
    a = np.arange(1, 7, dtype=np.float32).reshape(2, 3)
    b = np.arange(1, 13, dtype=np.float32).reshape(3, 4)
    c = oracle.gemm(a, b)
    # Row 0 of A is (1,2,3); column 0 of B is (1,5,9): 1 + 10 + 27 = 38.
    assert c[0, 0] == 38.0
    # Row 1 of A is (4,5,6); column 3 of B is (4,8,12): 16 + 40 + 72 = 128.
    assert c[1, 3] == 128.0
    assert c.tolist() == _exact_int_product(a, b)


# P2: identity.
@pytest.mark.parametrize("shape", [(1, 1), (17, 33), (64, 64), (97, 129), (300, 257)])
def test_identity_is_exact(shape):
    M, K = shape
    rng = np.random.default_rng(M * 1000 + K)
    a = rng.standard_normal((M, K), dtype=np.float32)
    b = rng.uniform(-1, 1, (M, K)).astype(np.float32)
    assert np.array_equal(oracle.gemm(a, np.eye(K, dtype=np.float32)), a)
    assert np.array_equal(oracle.gemm(np.eye(M, dtype=np.float32), b), b)


def test_identity_on_ragged_workload_rows():
    """A (first 64 rows of the ragged workload's A, K = 2049) x I_2049 = A exactly."""
    _, a, _ = make_workload("ragged")
    a = np.ascontiguousarray(a[:64])
    c = oracle.gemm(a, np.eye(a.shape[1], dtype=np.float32))
    assert np.array_equal(c, a)


# P3: all-ones.
@pytest.mark.parametrize("M,N,K", [(5, 7, 1), (33, 65, 257), (65, 33, 2049), (8, 8, 4096)])
def test_all_ones_gives_K(M, N, K):
    c = oracle.gemm(np.ones((M, K), np.float32), np.ones((K, N), np.float32))
    assert np.all(c == np.float32(K))


def test_all_ones_on_ragged_shape_sampled():
    M, N, K = 4097, 4095, 2049
    a = np.ones((M, K), np.float32)
    b = np.ones((K, N), np.float32)
    rng = np.random.default_rng(0)
    ii = np.concatenate([[0, M - 1, M - 1, 0], rng.integers(0, M, 500)])
    jj = np.concatenate([[0, N - 1, 0, N - 1], rng.integers(0, N, 500)])
    assert np.all(oracle.gemm_elems(a, b, ii, jj) == np.float32(K))


# P4: the 8x8, T = 4 block decomposition printed on page 3.
def test_block_decomposition_8x8_T4():
    with open(GOLDEN) as f:
        g = json.load(f)["block_decomposition"]
    n, t = g["N"], g["T"]
    rng = np.random.default_rng(42)
    a = rng.integers(-7, 8, (n, n)).astype(np.float32)
    b = rng.integers(-7, 8, (n, n)).astype(np.float32)
    c = oracle.gemm(a, b)

    def blk(x, name):
        r, s = int(name[1]), int(name[2])
        return np.ascontiguousarray(x[r * t:(r + 1) * t, s * t:(s + 1) * t])

    assert n // t == g["phases"]
    for cname, terms in g["terms"].items():
        acc = np.zeros((t, t), np.float32)
        for aname, bname in terms:
            acc = acc + oracle.gemm(blk(a, aname), blk(b, bname))
        assert np.array_equal(blk(c, cname), acc), cname


# P5: integer exactness on the 1024^3 integer workload (every partial sum < 2^24).
def test_integer_workload_exact():
    w, a, b = make_workload("square_1024_int")
    assert w.dist == "int4"
    c = oracle.gemm(a, b)
    exact = a.astype(np.int64) @ b.astype(np.int64)
    assert np.abs(exact).max() <= 16 * 1024
    assert np.array_equal(c.astype(np.int64), exact)


# P6: fp64 BLAS witness, within one fp32 ulp.
def _ulp_diff(x: np.ndarray, y: np.ndarray) -> np.ndarray:
    xi = x.astype(np.float32).view(np.int32).astype(np.int64)
    yi = y.astype(np.float32).view(np.int32).astype(np.int64)
    # map sign-magnitude to a monotone integer line
    xi = np.where(xi < 0, -(xi & 0x7FFFFFFF), xi)
    yi = np.where(yi < 0, -(yi & 0x7FFFFFFF), yi)
    return np.abs(xi - yi)


def test_blas_witness_square_256_full():
    w, a, b = make_workload("square_256")
    c = oracle.gemm(a, b)
    ref = (a.astype(np.float64) @ b.astype(np.float64)).astype(np.float32)
    d = _ulp_diff(c, ref)
    assert d.max() <= 1
    assert np.count_nonzero(d) <= c.size // 1000


@pytest.mark.parametrize("name", ["square_4096", "ragged", "skinny_k64"])
def test_blas_witness_sampled_large(name):
    w, a, b = make_workload(name)
    rng = np.random.default_rng(99)
    ii = np.concatenate([[0, w.M - 1], rng.integers(0, w.M, 2000)])
    jj = np.concatenate([[w.N - 1, 0], rng.integers(0, w.N, 2000)])
    got = oracle.gemm_elems(a, b, ii, jj)
    ref = np.einsum("tk,kt->t", a[ii].astype(np.float64), b[:, jj].astype(np.float64))
    d = _ulp_diff(got, ref.astype(np.float32))
    assert d.max() <= 1
    # Row and column bands through the full-matrix routine agree with the element routine.
    band = oracle.gemm(np.ascontiguousarray(a[:3]), b)
    assert np.array_equal(band[0, jj[:50]], oracle.gemm_elems(a, b, np.zeros(50, np.int64), jj[:50]))


# P7: accuracy against the correctly rounded sum, and the Higham bound.
def test_within_half_ulp_of_exact_sum():
    """fp64 accumulation keeps the oracle within (about) half an fp32 ulp of the
    exact sum.  A drop to fp32 accumulation breaks this on K = 4096."""
    rng = np.random.default_rng(5)
    M, N, K = 4, 5, 4096
    a = rng.uniform(-1, 1, (M, K)).astype(np.float32)
    b = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    c = oracle.gemm(a, b)
    for i in range(M):
        for j in range(N):
            terms = [float(a[i, k]) * float(b[k, j]) for k in range(K)]
            exact = math.fsum(terms)          # correctly rounded fp64 of the exact sum
            abs_sum = math.fsum(abs(t) for t in terms)
            ulp32 = float(np.spacing(np.float32(abs(exact))))
            slack = 0.5 * ulp32 + 2 * K * 2.0 ** -53 * abs_sum
            assert abs(float(c[i, j]) - exact) <= slack, (i, j)


def test_higham_bound_on_float_workload():
    """|C - exact| <= gamma_K (|A||B|) elementwise, the bound for any order."""
    w, a, b = make_workload("square_256")
    c = oracle.gemm(a, b).astype(np.float64)
    exact = a.astype(np.float64) @ b.astype(np.float64)
    bound = oracle.model.higham_gamma(w.K) * (np.abs(a).astype(np.float64) @ np.abs(b).astype(np.float64))
    assert np.all(np.abs(c - exact) <= bound + 1e-300)


# Leading dimensions, empty cases, C outside M x N untouched.
def test_leading_dimensions_and_padding_untouched():
    rng = np.random.default_rng(11)
    M, N, K = 7, 9, 5
    lda, ldb, ldc = 8, 13, 11
    a = rng.integers(-5, 6, (M, K)).astype(np.float32)
    b = rng.integers(-5, 6, (K, N)).astype(np.float32)
    abuf = np.full(M * lda, np.nan, np.float32)
    bbuf = np.full(K * ldb, np.nan, np.float32)
    for i in range(M):
        abuf[i * lda:i * lda + K] = a[i]
    for k in range(K):
        bbuf[k * ldb:k * ldb + N] = b[k]
    cbuf = np.full(M * ldc, -123.0, np.float32)
    oracle.gemm_ld(M, N, K, abuf, lda, bbuf, ldb, cbuf, ldc)
    exact = _exact_int_product(a, b)
    for i in range(M):
        assert cbuf[i * ldc:i * ldc + N].tolist() == exact[i]
        assert np.all(cbuf[i * ldc + N:(i + 1) * ldc] == -123.0)


def test_empty_cases():
    assert oracle.gemm(np.zeros((0, 4), np.float32), np.zeros((4, 3), np.float32)).shape == (0, 3)
    assert oracle.gemm(np.zeros((3, 4), np.float32), np.zeros((4, 0), np.float32)).shape == (3, 0)
    c = oracle.gemm(np.zeros((3, 0), np.float32), np.zeros((0, 5), np.float32))
    assert c.shape == (3, 5) and np.all(c == 0.0)


def test_bad_arguments_rejected():
    with pytest.raises(ValueError):
        oracle.gemm(np.zeros((2, 3), np.float32), np.zeros((4, 2), np.float32))
    with pytest.raises(ValueError):
        oracle.gemm_ld(2, 2, 3, np.zeros(6, np.float32), 2, np.zeros(6, np.float32), 2,
                       np.zeros(4, np.float32), 2)  # lda < K
    with pytest.raises(ValueError):
        oracle.gemm_elems(np.ones((2, 2), np.float32), np.ones((2, 2), np.float32), [2], [0])


def test_ieee_propagation():
    a = np.array([[np.inf, 1.0], [1.0, 1.0]], np.float32)
    b = np.array([[0.0, 1.0], [1.0, 1.0]], np.float32)
    c = oracle.gemm(a, b)
    assert np.isnan(c[0, 0])         # inf * 0
    assert c[0, 1] == np.inf
    assert c[1].tolist() == [1.0, 2.0]


# Planted mistakes: each is made in a copy of the data, on the CPU, and must be caught.
def test_planted_mistakes_are_caught():
    rng = np.random.default_rng(3)
    a = rng.integers(-4, 5, (6, 5)).astype(np.float32)
    b = rng.integers(-4, 5, (5, 4)).astype(np.float32)
    exact = np.array(_exact_int_product(a, b), np.float32)
    assert np.array_equal(oracle.gemm(a, b), exact)
    # dropped last term
    assert not np.array_equal(oracle.gemm(np.ascontiguousarray(a[:, :-1]),
                                          np.ascontiguousarray(b[:-1])), exact)
    # wrong sign
    assert not np.array_equal(oracle.gemm(-a, b), exact)
    # transposed operand in a square case
    sq = rng.integers(-4, 5, (5, 5)).astype(np.float32)
    assert not np.array_equal(oracle.gemm(np.ascontiguousarray(sq.T), b),
                              np.array(_exact_int_product(sq, b), np.float32))
    # fp32 accumulation misses the half-ulp pin above on long sums
    r = np.random.default_rng(5)
    K = 4096
    violations = 0
    for _ in range(8):
        x = r.uniform(-1, 1, K).astype(np.float32)
        y = r.uniform(-1, 1, K).astype(np.float32)
        acc32 = np.float32(0)
        for k in range(K):
            acc32 = np.float32(acc32 + np.float32(x[k] * y[k]))
        terms = [float(x[k]) * float(y[k]) for k in range(K)]
        exact_sum = math.fsum(terms)
        slack = 0.5 * float(np.spacing(np.float32(abs(exact_sum)))) + 2 * K * 2.0 ** -53 * math.fsum(map(abs, terms))
        violations += abs(float(acc32) - exact_sum) > slack
        assert abs(float(oracle.gemm(x.reshape(1, K), y.reshape(K, 1))[0, 0]) - exact_sum) <= slack
    assert violations >= 1
