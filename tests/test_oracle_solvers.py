"""Pins of the oracle's Krylov solvers (conjugate gradients, BiCGSTAB) by
exact-arithmetic facts and by dense solves:

* CG terminates in one step on the identity and on an eigenvector of A, and
  in as many steps as A has distinct eigenvalues (diagonal A);
* CG and BiCGSTAB agree with numpy.linalg.solve on small SPD and
  nonsymmetric matrices;
* the 5-point Laplacian (C1) is solved to the requested residual;
* an iteration cap is honoured and reported.
"""
import math

import numpy as np
import pytest

import oracle
from gen import CSR, c1_laplace2d, random_csr


def dense_to_csr(D):
    n = D.shape[0]
    rows, cols = np.nonzero(D)
    rowptr = np.concatenate([[0], np.cumsum(np.bincount(rows, minlength=n))]).astype(np.int64)
    return CSR(n, rowptr, cols.astype(np.int32), D[rows, cols].astype(np.float64))


def test_cg_identity_one_step():
    n = 50
    a = dense_to_csr(np.eye(n))
    b = np.random.default_rng(1).standard_normal(n)
    x, it, rel = oracle.cg(a, b, rtol=1e-14)
    assert it == 1 and np.allclose(x, b, rtol=0, atol=1e-15)


def test_cg_distinct_eigenvalues():
    # diagonal with 3 distinct values: the Krylov space has dimension 3
    d = np.array([1.0, 4.0, 9.0] * 20)
    a = dense_to_csr(np.diag(d))
    b = np.random.default_rng(2).standard_normal(d.size)
    x, it, rel = oracle.cg(a, b, rtol=1e-12)
    assert it == 3 and rel <= 1e-12
    assert np.allclose(x, b / d, rtol=1e-12, atol=0)


def test_cg_laplacian_eigenvector():
    a = c1_laplace2d()   # 64 x 64 grid, eigenvectors are products of sines
    r, c = np.divmod(np.arange(a.n), 64)
    v = np.sin(2 * math.pi * (r + 1) / 65) * np.sin(3 * math.pi * (c + 1) / 65)
    lam = 4 - 2 * math.cos(2 * math.pi / 65) - 2 * math.cos(3 * math.pi / 65)
    x, it, rel = oracle.cg(a, v, rtol=1e-12)
    assert it == 1
    assert np.allclose(x, v / lam, rtol=0, atol=1e-12)


def test_cg_random_spd_matches_dense_solve():
    rng = np.random.default_rng(3)
    B = rng.standard_normal((80, 80)) * (rng.random((80, 80)) < 0.1)
    A = B @ B.T + 80 * np.eye(80)
    a = dense_to_csr(A)
    b = rng.standard_normal(80)
    x, it, rel = oracle.cg(a, b, rtol=1e-13)
    assert rel <= 1e-13 and it <= 80
    assert np.allclose(x, np.linalg.solve(A, b), rtol=1e-10, atol=0)


def test_bicgstab_nonsymmetric_matches_dense_solve():
    rng = np.random.default_rng(4)
    A = rng.standard_normal((90, 90)) * (rng.random((90, 90)) < 0.08) + 6 * np.eye(90)
    a = dense_to_csr(A)
    b = rng.standard_normal(90)
    x, it, rel = oracle.bicgstab(a, b, rtol=1e-12)
    assert rel <= 1e-12
    assert np.allclose(x, np.linalg.solve(A, b), rtol=1e-9, atol=0)
    x1, it1, _ = oracle.bicgstab(dense_to_csr(np.eye(10)), np.arange(1.0, 11.0), rtol=1e-14)
    assert it1 == 1 and np.allclose(x1, np.arange(1.0, 11.0), rtol=0, atol=1e-15)


def test_laplacian_solve_and_cap():
    a = c1_laplace2d()
    x_true = np.random.default_rng(5).standard_normal(a.n)
    b = oracle.spmv(a, x_true)[0]
    x, it, rel = oracle.cg(a, b, rtol=1e-10, max_iter=2000)
    assert rel <= 1e-10
    assert np.linalg.norm(x - x_true) <= 1e-6 * np.linalg.norm(x_true)
    x2, it2, rel2 = oracle.bicgstab(a, b, rtol=1e-10, max_iter=2000)
    assert rel2 <= 1e-10 and np.linalg.norm(x2 - x_true) <= 1e-6 * np.linalg.norm(x_true)
    x3, it3, rel3 = oracle.cg(a, b, rtol=1e-10, max_iter=5)
    assert it3 == 5 and rel3 > 1e-10
    # a zero right-hand side needs no iteration
    x4, it4, rel4 = oracle.cg(a, np.zeros(a.n), rtol=1e-10)
    assert it4 == 0 and not np.any(x4)
