"""Pins of the oracle's reference converters (ELLPACK-R, SELL-64, HYB/HEC).

Slot counts are checked against the closed forms of "Sparse matrix-vector
multiplication on GPGPU clusters" (Sect. 2.1-2.2: N x Nmax for ELLPACK with N
padded to the SIMD width; (b_r + 1) N - b_r for pJDS in the one-full-row
case; no overhead at constant row length), every layout is decoded back to
the input CSR bit for bit by code written here, and the HYB/HEC width rule is
checked on hand-counted examples.
"""
import os

import numpy as np
import pytest

import oracle
from gen import CSR, c1_laplace2d, random_csr, stencil

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def read_kv(name):
    out = {}
    for line in open(os.path.join(GOLD, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            out[k] = int(v)
    return out


def one_full_row(N, full=0):
    lens = np.ones(N, dtype=np.int64)
    lens[full] = N
    rowptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    col = np.concatenate([np.arange(N) if i == full else [i] for i in range(N)]).astype(np.int32)
    return CSR(N, rowptr, col, np.arange(1, rowptr[-1] + 1, dtype=np.float64))


def ell_to_csr(n, oc, ov, ol, block=0):
    B = oracle.pad64(n) if block <= 0 else block
    W = oc.size // max(ol.size, 1)
    rows_c, rows_v = [], []
    for i in range(n):
        idx = (i // B) * W * B + np.arange(ol[i]) * B + i % B
        rows_c.append(oc[idx])
        rows_v.append(ov[idx])
    return rows_c, rows_v


def sell_to_csr(n, perm, sp, ls, oc, ov):
    rows_c = [None] * n
    rows_v = [None] * n
    for r in range(n):
        idx = sp[r // 64] + 64 * np.arange(ls[r]) + r % 64
        rows_c[perm[r]] = oc[idx]
        rows_v[perm[r]] = ov[idx]
    return rows_c, rows_v


def same_rows(a, rows_c, rows_v):
    for i in range(a.n):
        s, e = a.rowptr[i], a.rowptr[i + 1]
        assert np.array_equal(rows_c[i], a.col[s:e])
        assert rows_v[i].tobytes() == a.val[s:e].tobytes()


MATS = [
    ("c1", lambda: c1_laplace2d()),
    ("rand_ragged", lambda: random_csr(1000, seed=31, density=0.01, empty_frac=0.2,
                                       long_rows=3, long_len=700)),
    ("rand_dups_unsorted", lambda: random_csr(129, seed=32, density=0.05, dup_frac=0.3,
                                              zero_frac=0.1, unsorted=True)),
    ("fp32", lambda: random_csr(300, seed=33, density=0.03, dtype=np.float32)),
    ("n1", lambda: CSR(1, np.array([0, 3], np.int64), np.array([0, 0, 0], np.int32),
                       np.array([1.0, -0.0, 2.0]))),
    ("nnz0", lambda: CSR(65, np.zeros(66, np.int64), np.zeros(0, np.int32), np.zeros(0))),
]


def test_ell_slot_counts_closed_form():
    a = c1_laplace2d()
    oc, ov, ol = oracle.ell(a)
    assert oc.size == 20480 == 64 * 64 * 5
    # 27-point stencil on 128^3 (sizes only, from the closed form)
    assert oracle.pad64(128 ** 3) * 27 == 56_623_104


def test_pjds_worst_case_fixture():
    g = read_kv("p1_pjds_worst_case.txt")
    N, br = g["N"], g["b_r"]
    a = one_full_row(N)
    oc, _, _ = oracle.ell(a)
    assert oc.size == g["ell_slots"] == N * N
    perm, sp, ls, sc, _ = oracle.sell(a)
    assert sc.size == g["sell_slots"] == (br + 1) * N - br
    # the full row sorts first
    assert perm[0] == 0


def test_constant_length_has_no_padding():
    n, L = 256, 7
    lens = np.full(n, L)
    a = random_csr(n, seed=34, lens=lens)
    assert oracle.ell(a)[0].size == a.nnz
    assert oracle.sell(a)[3].size == a.nnz


def test_sell_slot_counts_stencils():
    a = c1_laplace2d()
    assert oracle.sell(a)[3].size == 20288
    # 27-point stencil: the sorted layout pads only inside mixed slices
    b = stencil((16, 16, 16), "box", 26.0, -1.0)
    perm, sp, ls, sc, _ = oracle.sell(b)
    L = np.sort(b.row_lengths())[::-1]
    Lp = np.concatenate([L, np.zeros(oracle.pad64(b.n) - b.n, L.dtype)])
    assert sc.size == int(sum(64 * Lp[s * 64] for s in range(Lp.size // 64)))


@pytest.mark.parametrize("name,mk", MATS)
def test_ell_round_trip(name, mk):
    a = mk()
    oc, ov, ol = oracle.ell(a)
    W = oracle.max_len(a)
    S = oracle.pad64(a.n)
    assert oc.size == W * S and ol.size == S
    assert np.all(ol[a.n:] == 0)
    same_rows(a, *ell_to_csr(a.n, oc, ov, ol))
    # pads are column 0 / +0.0
    used = np.zeros(W * S, bool)
    for i in range(a.n):
        used[np.arange(ol[i]) * S + i] = True
    assert np.all(oc[~used] == 0)
    assert ov[~used].tobytes() == np.zeros((~used).sum(), ov.dtype).tobytes()


def test_blocked_ell_layout_small():
    """Blocks of B rows, each column-major: hand-placed 5-row example, B = 2."""
    a = CSR(5, np.array([0, 2, 3, 3, 6, 7], np.int64), np.array([4, 1, 0, 2, 3, 4, 1], np.int32),
            np.arange(1.0, 8.0))
    oc, ov, ol = oracle.ell(a, 3, block=2)
    # padded rows R = 6, width 3: block k holds rows 2k, 2k+1, slot j*2 + r
    assert list(ol) == [2, 1, 0, 3, 1, 0]
    assert list(ov) == [1, 3, 2, 0, 0, 0,  0, 4, 0, 5, 0, 6,  7, 0, 0, 0, 0, 0]
    assert list(oc) == [4, 0, 1, 0, 0, 0,  0, 2, 0, 3, 0, 4,  1, 0, 0, 0, 0, 0]


@pytest.mark.parametrize("name,mk", MATS)
def test_sell_round_trip(name, mk):
    a = mk()
    perm, sp, ls, oc, ov = oracle.sell(a)
    L = a.row_lengths()
    # perm is a bijection sorted by (length desc, row asc)
    assert np.array_equal(np.sort(perm), np.arange(a.n))
    key = list(zip(-L[perm], perm))
    assert key == sorted(key)
    assert np.array_equal(ls[:a.n], L[perm]) and np.all(ls[a.n:] == 0)
    widths = np.diff(sp) // 64
    assert np.all(np.diff(sp) % 64 == 0)
    assert np.array_equal(widths, ls[::64])
    same_rows(a, *sell_to_csr(a.n, perm, sp, ls, oc, ov))


def test_hyb_width_fixture():
    for line in open(os.path.join(GOLD, "hyb_width_examples.txt")):
        if line.startswith("#") or not line.strip():
            continue
        k, lens = line.split("|")
        lens = np.array([int(v) for v in lens.split()], dtype=np.int64)
        a = random_csr(lens.size, seed=1, lens=lens)
        assert oracle.hyb_width(a) == int(k), (k, lens)


def test_regular_width_examples():
    """Hand-counted: the smallest k with at most 1 % of the rows longer."""
    def mk(lens):
        lens = np.asarray(lens, np.int64)
        rp = np.concatenate([[0], np.cumsum(lens)])
        return CSR(len(lens), rp, np.zeros(rp[-1], np.int32), np.ones(rp[-1]))
    assert oracle.regular_width(mk([1] * 99 + [50])) == 1       # one row of 100 may be longer
    assert oracle.regular_width(mk([1] * 98 + [50, 50])) == 50  # two may not
    assert oracle.regular_width(mk([3] * 100)) == 3
    assert oracle.regular_width(mk([0] * 10)) == 0
    assert oracle.regular_width(mk([])) == 0
    assert oracle.regular_width(mk([5, 1, 1])) == 5             # n < 100: no row may be longer
    lens = [20 + i % 21 for i in range(2000)]                   # 20..40, as in the FEM block
    for i in range(0, 2000, 100):
        lens[i] = 2000                                          # exactly 1 % long rows
    assert oracle.regular_width(mk(lens)) == 40
    assert oracle.hyb_width(mk(lens)) < 40


def test_hyb_width_stencils_and_override():
    a = c1_laplace2d()
    assert oracle.hyb_width(a) == 5
    b = stencil((12, 12, 12), "box", 26.0, -1.0)
    assert oracle.hyb_width(b) == 27
    assert oracle.hyb_width(a, 20) == 5      # clamped to the longest row
    assert oracle.hyb_width(a, 3) == 3
    assert oracle.hyb_width(a, 0) == 0


@pytest.mark.parametrize("name,mk", MATS)
@pytest.mark.parametrize("K", [0, 1, 3, None, 10 ** 6])
def test_split_round_trip(name, mk, K):
    """ELL part (width K) + tail (COO and CSR) rebuild the input exactly."""
    a = mk()
    K = oracle.hyb_width(a) if K is None else oracle.hyb_width(a, K)
    B = oracle.ELL_BLOCK_SPLIT
    oc, ov, ol = oracle.ell(a, K, block=B)
    L = a.row_lengths()
    assert ol.size == -(-a.n // B) * B and oc.size == K * ol.size
    assert np.array_equal(ol[:a.n], np.minimum(L, K)) and np.all(ol[a.n:] == 0)
    trow, tptr, tcol, tval = oracle.tail(a, K)
    assert trow.size == int(np.maximum(L - K, 0).sum())
    assert np.array_equal(np.diff(tptr), np.maximum(L - K, 0))
    assert np.all(np.diff(trow) >= 0)
    ec, ev = ell_to_csr(a.n, oc, ov, ol, block=B)
    rows_c, rows_v = [], []
    for i in range(a.n):
        sel = slice(tptr[i], tptr[i + 1])
        assert np.all(trow[sel] == i)
        rows_c.append(np.concatenate([ec[i], tcol[sel]]))
        rows_v.append(np.concatenate([ev[i], tval[sel]]))
    same_rows(a, rows_c, rows_v)


def _hand5():
    # lengths 2, 1, 0, 3, 1
    return CSR(5, np.array([0, 2, 3, 3, 6, 7], np.int64), np.array([4, 1, 0, 2, 3, 4, 1], np.int32),
               np.arange(1.0, 8.0))


def test_sorted_ell_layout_small():
    """Windowed sort of the blocked ELL part, hand-placed: B = 4, W = 3."""
    a = _hand5()
    oc, ov, ol, op = oracle.ell(a, 3, block=4, sigma=4, with_perm=True)
    # block 0 holds rows 0..3 ordered by length desc: 3, 0, 1, 2; block 1: row 4 + padding
    assert list(op) == [3, 0, 1, 2, 4, 5, 6, 7]
    assert list(ol) == [3, 2, 1, 0, 1, 0, 0, 0]
    assert list(ov) == [4, 1, 3, 0, 5, 2, 0, 0, 6, 0, 0, 0,  7] + [0] * 11
    assert list(oc) == [2, 4, 0, 0, 3, 1, 0, 0, 4, 0, 0, 0,  1] + [0] * 11
    # windows of 2 positions: {0, 1} keeps rows 0, 1; {2, 3} puts row 3 first
    oc, ov, ol, op = oracle.ell(a, 3, block=4, sigma=2, with_perm=True)
    assert list(op[:4]) == [0, 1, 3, 2] and list(ol[:4]) == [2, 1, 3, 0]
    assert list(ov[:12]) == [1, 3, 4, 0, 2, 0, 5, 0, 0, 0, 6, 0]
    assert list(oc[:12]) == [4, 0, 2, 0, 1, 0, 3, 0, 0, 0, 4, 0]
    # sigma 0 is the unsorted layout
    u = oracle.ell(a, 3, block=4, with_perm=True)
    assert list(u[3]) == list(range(8))


@pytest.mark.parametrize("name,mk", MATS)
@pytest.mark.parametrize("sigma", [64, 256, 1024])
def test_sorted_ell_round_trip(name, mk, sigma):
    a = mk()
    B = oracle.ELL_BLOCK_SPLIT
    K = oracle.hyb_width(a)
    oc, ov, ol, op = oracle.ell(a, K, block=B, sigma=sigma, with_perm=True)
    R = ol.size
    assert np.array_equal(np.sort(op), np.arange(R))
    assert np.array_equal(op[a.n:], np.arange(a.n, R))
    L = np.minimum(a.row_lengths(), K)
    assert np.array_equal(ol[:a.n], L[op[:a.n]])
    # inside every window: stored length descending, then row ascending
    for w0 in range(0, a.n, sigma):
        rows = op[w0:min(w0 + sigma, a.n)]
        assert np.all((rows >= w0) & (rows < w0 + sigma))
        key = list(zip(-L[rows], rows))
        assert key == sorted(key)
    # decode by position, then undo the permutation
    pc, pv = ell_to_csr(R, oc, ov, ol, block=B)
    rows_c, rows_v = [None] * a.n, [None] * a.n
    for p in range(a.n):
        rows_c[op[p]], rows_v[op[p]] = pc[p], pv[p]
    for i in range(a.n):
        s = a.rowptr[i]
        assert np.array_equal(rows_c[i], a.col[s:s + L[i]])
        assert rows_v[i].tobytes() == a.val[s:s + L[i]].tobytes()


def test_ell_pad_fraction():
    a = _hand5()
    # one wave of 64 rows runs to the longest stored row (3): 64 * 3 slots for 7 entries
    assert oracle.ell_pad_fraction(a, 3) == pytest.approx(1 - 7 / 192)
    assert oracle.ell_pad_fraction(a, 1) == pytest.approx(1 - 4 / 64)
    # constant length over whole waves reads no padding
    b = random_csr(256, seed=35, lens=np.full(256, 9))
    assert oracle.ell_pad_fraction(b, 9) == 0.0
    assert oracle.ell_pad_fraction(b, 20) == 0.0
    # two waves: lengths 1 and 5 alternating in the first, all 2 in the second
    lens = np.concatenate([np.tile([1, 5], 32), np.full(64, 2)])
    c = random_csr(128, seed=36, lens=lens)
    assert oracle.ell_pad_fraction(c, 8) == pytest.approx(1 - (32 * 6 + 128) / (64 * 5 + 64 * 2))


def test_sell_windowed_sort():
    a = _hand5()
    perm, sp, ls, sc, sv = oracle.sell(a, sigma=2)
    assert list(perm) == [0, 1, 3, 2, 4]
    # one slice, padded to its longest row (3), not to its first row
    assert list(sp) == [0, 192] and list(ls[:5]) == [2, 1, 3, 0, 1]
    same_rows(a, *sell_to_csr(a.n, perm, sp, ls, sc, sv))
    ident = oracle.sell(a, sigma=1)[0]
    assert list(ident) == list(range(5))
    b = random_csr(1000, seed=37, density=0.01, empty_frac=0.2, long_rows=3, long_len=700)
    whole = oracle.sell(b)
    for sigma in (b.n, 4096):
        w = oracle.sell(b, sigma=sigma)
        assert all(np.array_equal(u, v) for u, v in zip(whole, w))
    perm, sp, ls, sc, sv = oracle.sell(b, sigma=128)
    L = b.row_lengths()
    for w0 in range(0, b.n, 128):
        rows = perm[w0:w0 + 128]
        assert np.all((rows >= w0) & (rows < w0 + 128))
        key = list(zip(-L[rows], rows))
        assert key == sorted(key)
    widths = np.diff(sp) // 64
    Lp = np.concatenate([L[perm], np.zeros(oracle.pad64(b.n) - b.n, np.int64)])
    assert np.array_equal(widths, Lp.reshape(-1, 64).max(axis=1))
    same_rows(b, *sell_to_csr(b.n, perm, sp, ls, sc, sv))


def test_sell_permuted_basis():
    """Permuted basis: row r of P A P^T is row perm[r] of A with every column c
    replaced by its sorted position (hand example, then a round trip)."""
    a = _hand5()   # lengths 2, 1, 0, 3, 1; sorted: 3, 0, 1, 4, 2
    perm, sp, ls, sc, sv = oracle.sell(a, permuted=True)
    assert list(perm) == [3, 0, 1, 4, 2]
    inv = {int(p): r for r, p in enumerate(perm)}
    # sorted positions: row 3 -> 0, 0 -> 1, 1 -> 2, 4 -> 3, 2 -> 4
    assert inv == {3: 0, 0: 1, 1: 2, 4: 3, 2: 4}
    # row 3 of A (lane 0): cols 2, 3, 4 -> 4, 0, 3 in columns 0..2 of the slice
    assert [sc[0], sc[64], sc[128]] == [4, 0, 3]
    # row 0 (lane 1): cols 4, 1 -> 3, 2; row 1 (lane 2): col 0 -> 1; row 4 (lane 3): col 1 -> 2
    assert [sc[1], sc[65], sc[2], sc[3]] == [3, 2, 1, 2]
    plain = oracle.sell(a)
    assert sv.tobytes() == plain[4].tobytes() and np.array_equal(sp, plain[1])
    b = random_csr(1000, seed=38, density=0.01, empty_frac=0.2, long_rows=3, long_len=700)
    perm, sp, ls, sc, sv = oracle.sell(b, sigma=128, permuted=True)
    rows_c, rows_v = sell_to_csr(b.n, perm, sp, ls, sc, sv)
    # undo the renumbering: sorted position -> original row
    same_rows(b, [perm[c] for c in rows_c], rows_v)
    # the permuted product equals the permuted original product
    x = np.random.default_rng(3).standard_normal(b.n)
    y = oracle.spmv(b, x)[0]
    # rows_c / rows_v are indexed by original row: row r of P A P^T is row perm[r]
    A_perm = CSR(b.n, np.concatenate([[0], np.cumsum(b.row_lengths()[perm])]).astype(np.int64),
                 np.concatenate([rows_c[p] for p in perm]).astype(np.int32),
                 np.concatenate([rows_v[p] for p in perm]))
    yp = oracle.spmv(A_perm, x[perm])[0]
    assert np.allclose(yp, y[perm], rtol=0, atol=1e-12 * np.abs(y).max())
