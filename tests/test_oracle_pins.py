"""Pins of the CPU oracle's SpMV against things other than itself.

Each test checks the oracle against a value fixed by mathematics or by the
pages: exact rational arithmetic, a densified matvec, correctly rounded row
sums, closed-form eigen-relations of stencil matrices, and special cases.
A plausible slip in the oracle (a dropped compensation term, a wrong sign on
beta, a transposed operand, an off-by-one row range) fails at least one.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from gen import (CSR, c1_laplace2d, random_csr, stencil, vectors)

EPS = 2.0 ** -53


def gamma(k):
    return k * EPS / (1 - k * EPS)


def exact_row(a, i, x):
    s = Fraction(0)
    for k in range(int(a.rowptr[i]), int(a.rowptr[i + 1])):
        s += Fraction(float(a.val[k])) * Fraction(float(x[a.col[k]]))
    return s


def cancel_matrix(n, seed, spread=150):
    """Rows whose products nearly cancel, with magnitudes 1e+-spread."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, 12, n)
    rowptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    nnz = int(rowptr[-1])
    col = rng.integers(0, n, nnz).astype(np.int32)
    val = np.empty(nnz)
    for i in range(n):
        s, e = rowptr[i], rowptr[i + 1]
        m = e - s
        big = rng.uniform(-1, 1, m) * 10.0 ** rng.integers(-spread, spread, m)
        val[s:e] = big
        if m >= 3:
            # pair a product with its negative plus a tiny remainder
            val[s + 1] = -val[s] * (1 + 2.0 ** -40)
    return CSR(n, rowptr, col, val)


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_dot2_against_exact_rationals(seed):
    """|y - exact| <= eps|exact| + gamma_n^2 sum|a x| (Dot2 error bound)."""
    n = 48
    a = cancel_matrix(n, seed)
    x = np.random.default_rng(100 + seed).uniform(-1, 1, n) * \
        10.0 ** np.random.default_rng(200 + seed).integers(-20, 20, n)
    y, sc = oracle.spmv(a, x)
    plain_fail = 0
    for i in range(n):
        ex = exact_row(a, i, x)
        m = int(a.rowptr[i + 1] - a.rowptr[i])
        absum = sum(abs(Fraction(float(a.val[k])) * Fraction(float(x[a.col[k]])))
                    for k in range(int(a.rowptr[i]), int(a.rowptr[i + 1])))
        bound = Fraction(EPS) * abs(ex) + Fraction(gamma(2 * m + 2)) ** 2 * absum * 4
        assert abs(Fraction(float(y[i])) - ex) <= bound, (i, float(y[i]), float(ex))
        # the same rows summed plainly miss this bound somewhere: the
        # compensation is what the test is sensitive to
        plain = 0.0
        for k in range(int(a.rowptr[i]), int(a.rowptr[i + 1])):
            plain += float(a.val[k]) * float(x[a.col[k]])
        if abs(Fraction(plain) - ex) > bound:
            plain_fail += 1
    assert plain_fail > 0


def test_alpha_beta_exact():
    """y = alpha * r + beta * y0 against exact rationals, both signs of beta."""
    a = random_csr(40, seed=5, density=0.2)
    x, y0 = vectors(40, 5)
    for alpha, beta in [(1.5, -0.5), (-1.0, 1.0), (0.0, 2.0), (2.0, 0.0)]:
        y, sc = oracle.spmv(a, x, y0, alpha, beta)
        for i in range(a.n):
            ex = Fraction(alpha) * exact_row(a, i, x) + Fraction(beta) * Fraction(float(y0[i]))
            assert abs(Fraction(float(y[i])) - ex) <= Fraction(4 * EPS) * Fraction(float(sc[i])) + \
                Fraction(1, 10 ** 300), (alpha, beta, i)


def test_scale_definition_hand_example():
    """The tolerance scale is |alpha| * sum |a x| + |beta * y0| (hand-computed):
    row [1, -2, 4] against x = [1, 1, 0.5] has sum |a x| = 1 + 2 + 2 = 5 and
    sum a x = 1; alpha = -3, beta = 0.5, y0 = -8 give y = -3 - 4 = -7 and a
    scale of 15 + 4 = 19."""
    a = CSR(3, np.array([0, 3, 3, 3], np.int64), np.array([0, 1, 2], np.int32),
            np.array([1.0, -2.0, 4.0]))
    x = np.array([1.0, 1.0, 0.5])
    y0 = np.array([-8.0, 6.0, 0.0])
    y, sc = oracle.spmv(a, x, y0, -3.0, 0.5)
    assert y.tolist() == [-7.0, 3.0, 0.0]
    assert sc.tolist() == [19.0, 3.0, 0.0]
    y, sc = oracle.spmv(a, x, None, 2.0, 0.0)   # beta = 0: y0 is not read
    assert y.tolist() == [2.0, 0.0, 0.0] and sc.tolist() == [10.0, 0.0, 0.0]


@pytest.mark.parametrize("kw", [
    dict(n=150, seed=11, density=0.05),
    dict(n=200, seed=12, density=0.03, empty_frac=0.3, unsorted=True),
    dict(n=97, seed=13, density=0.1, dup_frac=0.3, zero_frac=0.2),
    dict(n=130, seed=14, density=0.02, long_rows=2, long_len=130),
])
def test_against_dense_matvec(kw):
    """Densified A (duplicates summed) times x, nonsymmetric matrices."""
    a = random_csr(**kw)
    x, y0 = vectors(a.n, kw["seed"])
    D = np.zeros((a.n, a.n))
    rows = np.repeat(np.arange(a.n), a.row_lengths())
    np.add.at(D, (rows, a.col), a.val)
    ref = D @ x * 1.25 - 0.75 * y0
    y, sc = oracle.spmv(a, x, y0, 1.25, -0.75)
    absx = np.abs(D) @ np.abs(x) * 1.25 + 0.75 * np.abs(y0)
    # duplicates pre-summed in D add one rounding per entry: 3 gamma_n covers it
    tol = 3 * gamma(a.n + 4) * absx + 1e-300
    assert np.all(np.abs(y - ref) <= tol)
    # the transpose differs (catches a swapped operand)
    assert not np.allclose(D.T @ x * 1.25 - 0.75 * y0, y, rtol=0, atol=1e-8)


def test_row_sums_correctly_rounded():
    """A * 1 equals the correctly rounded row sums (math.fsum)."""
    a = random_csr(300, seed=21, density=0.1)
    a.val *= 10.0 ** np.random.default_rng(3).integers(-8, 8, a.val.size)
    y, _ = oracle.spmv(a, np.ones(a.n))
    for i in range(a.n):
        s, e = a.rowptr[i], a.rowptr[i + 1]
        assert y[i] == math.fsum(a.val[s:e].tolist())


def test_laplace2d_closed_forms():
    """5-point Laplacian on 64^2: A 1 = 4 - degree; linear x is harmonic
    inside; sine modes are eigenvectors with 4 - 2cos(p pi/65) - 2cos(q pi/65)."""
    m = 64
    a = c1_laplace2d(m)
    assert a.n == 4096 and a.nnz == 20224
    r = np.arange(a.n) // m
    c = np.arange(a.n) % m
    deg = (r > 0).astype(int) + (r < m - 1) + (c > 0) + (c < m - 1)
    y, _ = oracle.spmv(a, np.ones(a.n))
    assert np.array_equal(y, 4.0 - deg)
    for xv in (r.astype(float), c.astype(float)):
        y, _ = oracle.spmv(a, xv)
        interior = (r > 0) & (r < m - 1) & (c > 0) & (c < m - 1)
        assert np.all(y[interior] == 0.0)
        assert np.any(y[~interior] != 0.0)
    for p, q in [(1, 1), (3, 7), (64, 2), (40, 41)]:
        v = np.sin(p * np.pi * (r + 1) / (m + 1)) * np.sin(q * np.pi * (c + 1) / (m + 1))
        lam = 4 - 2 * np.cos(p * np.pi / (m + 1)) - 2 * np.cos(q * np.pi / (m + 1))
        y, sc = oracle.spmv(a, v)
        assert np.max(np.abs(y - lam * v)) <= 1e-14 * np.max(sc) + 1e-15


def test_stencil27_closed_form():
    """27-point stencil with no noise: A 1 = 27 - len exactly, and the row
    length classes of an m^3 box stencil."""
    m = 20
    a = stencil((m, m, m), "box", 26.0, -1.0)
    L = a.row_lengths()
    y, _ = oracle.spmv(a, np.ones(a.n))
    assert np.array_equal(y, 27.0 - L)
    counts = {27: (m - 2) ** 3, 18: 6 * (m - 2) ** 2, 12: 12 * (m - 2), 8: 8}
    for k, v in counts.items():
        assert int(np.sum(L == k)) == v


def test_special_cases():
    rng = np.random.default_rng(7)
    n = 70
    x = rng.uniform(-1, 1, n)
    y0 = rng.uniform(-1, 1, n)
    eye = CSR(n, np.arange(n + 1, dtype=np.int64), np.arange(n, dtype=np.int32), np.ones(n))
    y, _ = oracle.spmv(eye, x)
    assert np.array_equal(y, x)
    d = rng.uniform(-3, 3, n)
    diag = CSR(n, np.arange(n + 1, dtype=np.int64), np.arange(n, dtype=np.int32), d)
    y, _ = oracle.spmv(diag, x)
    assert np.array_equal(y, d * x)
    a = random_csr(n, seed=8, density=0.1)
    y, _ = oracle.spmv(a, x, y0, 0.0, -2.5)
    assert np.array_equal(y, -2.5 * y0)
    empty = CSR(n, np.zeros(n + 1, dtype=np.int64), np.zeros(0, np.int32), np.zeros(0))
    y, sc = oracle.spmv(empty, x, y0, 3.0, 0.5)
    assert np.array_equal(y, 0.5 * y0)
    y, sc = oracle.spmv(empty, x)
    assert np.all(y == 0) and np.all(sc == 0)
    one = CSR(1, np.array([0, 2], dtype=np.int64), np.array([0, 0], np.int32), np.array([2.0, 3.0]))
    y, _ = oracle.spmv(one, np.array([0.5]))
    assert y[0] == 2.5
    # beta == 0 never reads y: NaN there stays out of the result
    y, _ = oracle.spmv(a, x, np.full(n, np.nan), 1.0, 0.0)
    assert np.all(np.isfinite(y))


def test_sampled_rows_match_full():
    a = random_csr(500, seed=9, density=0.02)
    x, y0 = vectors(a.n, 9)
    y, sc = oracle.spmv(a, x, y0, 0.5, 1.5)
    rows = np.array([499, 0, 17, 17, 250])
    ys, ss = oracle.spmv(a, x, y0, 0.5, 1.5, rows=rows)
    assert np.array_equal(ys, y[rows]) and np.array_equal(ss, sc[rows])


def test_threads_bit_identical():
    a = random_csr(3000, seed=10, density=0.01)
    x, _ = vectors(a.n, 10)
    y1, _ = oracle.spmv(a, x, nthreads=1)
    y4, _ = oracle.spmv(a, x, nthreads=4)
    assert np.array_equal(y1, y4)


def test_fp32_inputs_promote_exactly():
    a = random_csr(200, seed=15, density=0.05, dtype=np.float32)
    x = np.random.default_rng(1).uniform(-1, 1, a.n).astype(np.float32)
    y, _ = oracle.spmv(a, x)
    for i in range(0, a.n, 7):
        ex = exact_row(a, i, x.astype(np.float64))
        assert abs(Fraction(float(y[i])) - ex) <= Fraction(EPS) * abs(ex) + Fraction(1, 10 ** 200)


def test_check_rule():
    ok, worst, k = oracle.check(np.array([1.0, 0.0]), np.array([1.0 + 1e-13, 0.0]),
                                np.array([1.0, 0.0]), 1e-12)
    assert ok and k == 0
    ok, worst, k = oracle.check(np.array([1.0, 1e-300]), np.array([1.0, 0.0]),
                                np.array([1.0, 0.0]), 1e-12)
    assert not ok and k == 1
    ok, _, _ = oracle.check(np.array([np.nan]), np.array([1.0]), np.array([1.0]), 1e-12)
    assert not ok
