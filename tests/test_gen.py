"""Generator checks: determinism, the pages' printed sizes, workload statistics."""
import os

import numpy as np
import pytest

import gen
import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_poisson_nnz_fixture():
    """7-point Poisson sizes printed in the Krylov/AMG paper (Sect. 4)."""
    for line in open(os.path.join(GOLD, "p3_poisson_nnz.txt")):
        if line.startswith("#") or not line.strip():
            continue
        m, rows, nnz = (int(v) for v in line.split())
        assert m ** 3 == rows
        assert gen.stencil_nnz(m, 3, "star") == nnz
        if m <= 50:
            a = gen.stencil((m, m, m), "star", 6.0, -1.0)
            assert (a.n, a.nnz) == (rows, nnz)


def test_stencil_sizes():
    a = gen.c1_laplace2d()
    assert (a.n, a.nnz) == (4096, 20224) == (4096, gen.stencil_nnz(64, 2, "star"))
    assert gen.stencil_nnz(128, 3, "box") == 55_742_968
    b = gen.stencil((9, 9, 9), "box", 26.0, -1.0)
    assert b.nnz == gen.stencil_nnz(9, 3, "box")
    # columns strictly ascending inside rows, diagonal present
    rows = np.repeat(np.arange(b.n), b.row_lengths())
    key = rows.astype(np.int64) * b.n + b.col
    assert np.all(np.diff(key) > 0)
    assert np.sum(b.col == rows) == b.n


def test_determinism_small():
    a1 = gen.c5_fem(n=200_000, seed=77)
    a2 = gen.c5_fem(n=200_000, seed=77)
    assert a1.col.tobytes() == a2.col.tobytes() and a1.val.tobytes() == a2.val.tobytes()
    b1 = gen.c4_powerlaw(n=100_000, nlong=4, long_lo=2000, long_hi=5000, seed=78)
    b2 = gen.c4_powerlaw(n=100_000, nlong=4, long_lo=2000, long_hi=5000, seed=78)
    assert b1.col.tobytes() == b2.col.tobytes() and b1.val.tobytes() == b2.val.tobytes()
    x1, y1 = gen.vectors(1000, 5)
    x2, y2 = gen.vectors(1000, 5)
    assert np.array_equal(x1, x2) and np.array_equal(y1, y2) and not np.array_equal(x1, y1)


def test_fem_statistics_reduced():
    n = 400_000
    a = gen.c5_fem(n=n, seed=79)
    L = a.row_lengths()
    assert np.sum(L == 2000) == round(0.01 * n)
    short = L[L != 2000]
    assert short.min() == 20 and short.max() == 40
    rows = np.repeat(np.arange(n), L)
    key = rows.astype(np.int64) * n + a.col
    assert np.all(np.diff(key) > 0)           # sorted, no duplicates
    near = np.abs(a.col.astype(np.int64) - rows) <= 10_000
    assert 0.94 < near.mean() < 0.96
    assert abs(a.val.mean()) < 0.01 and abs(a.val.std() - 1) < 0.01


def test_hmep_statistics_reduced():
    """Bands in runs of 15,000 rows with gaps, mirrored (symmetric)."""
    n = 300_000
    a = gen.c2_hmep(n=n, dmax=100_000, seed=80)
    L = a.row_lengths()
    assert 10 < L.mean() < 20
    import scipy.sparse as sp
    m = sp.csr_matrix((a.val, a.col, a.rowptr), shape=(n, n))
    assert (m - m.T).count_nonzero() == 0
    assert np.all(m.diagonal() != 0)
    # every off-diagonal offset forms contiguous runs of 15,000 rows (or
    # runs cut by the matrix edge / phase at the start)
    rows = np.repeat(np.arange(n), L)
    off = a.col.astype(np.int64) - rows
    d = np.unique(off[off > 0])
    assert d.size == 14
    for dk in d[:3]:
        present = np.zeros(n, bool)
        present[rows[off == dk]] = True
        edges = np.flatnonzero(np.diff(present.astype(np.int8)))
        runs = np.diff(edges)
        assert np.all(runs[1:-1] % 5000 == 0)
        assert set(runs[1:-1].tolist()) <= {15_000, 10_000}


@pytest.mark.slow
def test_full_size_workloads():
    """Full sizes of the five workloads as drawn (realized nnz pinned so a
    generator change is noticed), plus the P1 HMEp shape."""
    a = gen.c2_hmep()
    L = a.row_lengths()
    assert a.n == 6_200_000 and a.nnz == 97_085_164
    assert 15 <= L.mean() <= 16 and L.max() == 22
    del a
    b = gen.c4_powerlaw()
    Lb = b.row_lengths()
    assert b.n == 4_000_000 and b.nnz == 42_193_576
    assert np.sum(Lb >= 20_000) == 64 and Lb.max() <= 50_000
    assert 10 < Lb.mean() < 11
    assert oracle.hyb_width(b) == 9


@pytest.mark.slow
def test_stencil27_full_size_layouts():
    """27-point stencil on 128^3: sizes of ELL-R and SELL-64 and the HYB width."""
    a = gen.c3_stencil27()
    assert (a.n, a.nnz) == (2_097_152, 55_742_968)
    L = a.row_lengths()
    counts = {27: 126 ** 3, 18: 6 * 126 ** 2, 12: 12 * 126, 8: 8}
    for k, v in counts.items():
        assert int(np.sum(L == k)) == v
    assert oracle.pad64(a.n) * int(L.max()) == 56_623_104
    Ls = np.sort(L)[::-1]
    assert int(sum(64 * Ls[s * 64] for s in range(a.n // 64))) == 55_743_360
    assert oracle.hyb_width(a) == 27
