"""Seeded synthetic sparse matrices and vectors.

This module only *draws* inputs: sparsity patterns, values, x and y0. It holds
none of the sparse matrix-vector arithmetic, so both the CPU oracle and the GPU
path can consume what it produces without sharing any of the method.

Every matrix comes out as CSR with int64 row pointers, int32 column indices
and float64 values (columns ascending inside a row unless a tiny test matrix
asks otherwise).  fp32 inputs are made by rounding the fp64 draws to nearest
(``as_fp32``); both sides then consume the rounded values.

Workloads (the shapes of the pages' matrices, drawn here since the originals
are not available):

* ``c1_laplace2d``  - 5-point Laplacian on a 64 x 64 grid (diag 4, off -1).
* ``c2_hmep``       - a Holstein-Hubbard-like banded symmetric matrix with
  n = 6.2e6 and about 15 entries per row made of contiguous off-diagonal runs
  of 15,000 rows (the HMEp description in "Sparse matrix-vector multiplication
  on GPGPU clusters", test matrices).
* ``c3_stencil27``  - 27-point stencil on a 128^3 grid (diag 26, neighbours
  -1 + 1e-3 N(0,1)).
* ``c4_powerlaw``   - 4e6 rows with lognormal row lengths (mean 10) plus 64
  rows of 20k-50k entries, uniform random columns.
* ``c5_fem``        - 8e6 rows of 20-40 entries plus 1% rows of 2,000 entries,
  95% of columns within +-10,000 of the diagonal.

Random streams: ``SeedSequence(1000 + k)`` for workload k spawns four
independent PCG64 streams (pattern, values, x, y0); the random column patterns
of the two irregular workloads draw from a fifth child, itself split into one
stream per chunk of rows so that chunks can be drawn in parallel.
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = [
    "CSR", "streams", "vectors", "as_fp32", "stencil", "c1_laplace2d",
    "c2_hmep", "c3_stencil27", "c4_powerlaw", "c5_fem", "random_csr",
    "stencil_nnz", "by_name", "WORKLOADS",
]


@dataclasses.dataclass
class CSR:
    n: int
    rowptr: np.ndarray   # int64[n+1]
    col: np.ndarray      # int32[nnz]
    val: np.ndarray      # float64[nnz] or float32[nnz]

    @property
    def nnz(self) -> int:
        return int(self.rowptr[-1])

    def row_lengths(self) -> np.ndarray:
        return np.diff(self.rowptr)


def streams(seed: int):
    """Four independent generators (pattern, values, x, y0) for one seed."""
    kids = np.random.SeedSequence(seed).spawn(4)
    return [np.random.Generator(np.random.PCG64(k)) for k in kids]


def vectors(n: int, seed: int, dtype=np.float64):
    """x ~ U[-1,1) and y0 ~ U[-1,1) of length n from the seed's x / y0 streams."""
    _, _, gx, gy = streams(seed)
    x = gx.uniform(-1.0, 1.0, n)
    y0 = gy.uniform(-1.0, 1.0, n)
    return x.astype(dtype), y0.astype(dtype)


def as_fp32(a: CSR) -> CSR:
    """Round values to fp32 (round to nearest even); the pattern is shared."""
    return CSR(a.n, a.rowptr, a.col, a.val.astype(np.float32))


def _from_table(n: int, mask: np.ndarray, cols: np.ndarray, vals: np.ndarray) -> CSR:
    """Compress (n, m) candidate tables, row-major, into CSR.

    Candidate j of row i is stored when ``mask[i, j]``; candidates are listed
    in ascending column order, so the CSR rows come out sorted.
    """
    lens = mask.sum(axis=1, dtype=np.int64)
    rowptr = np.zeros(n + 1, dtype=np.int64)
    np.cumsum(lens, out=rowptr[1:])
    return CSR(n, rowptr, cols[mask].astype(np.int32, copy=False), vals[mask])


# --------------------------------------------------------------------------
# stencils (5-point, 7-point, 27-point) on regular grids
# --------------------------------------------------------------------------

def stencil_offsets(ndim: int, kind: str):
    """Neighbour offsets in lexicographic order (ascending linear column)."""
    import itertools
    offs = []
    for t in itertools.product((-1, 0, 1), repeat=ndim):
        if kind == "star" and sum(abs(v) for v in t) > 1:
            continue
        offs.append(t)
    return offs


def stencil(dims, kind: str, diag: float, off: float, noise: float = 0.0,
            seed: int | None = None) -> CSR:
    """Stencil matrix on a grid with the last dimension fastest.

    kind "star" gives the (2d+1)-point stencil, "box" the 3^d-point one.
    Off-diagonal values are ``off + noise * N(0,1)``; the noise is drawn from
    the values stream as one length-n array per off-diagonal offset (in offset
    order) and read at the rows where that neighbour exists.  The diagonal is
    exactly ``diag``.
    """
    dims = tuple(int(d) for d in dims)
    nd = len(dims)
    n = int(np.prod(dims))
    offs = stencil_offsets(nd, kind)
    m = len(offs)
    strides = [int(np.prod(dims[k + 1:])) for k in range(nd)]
    t = np.array(offs, dtype=np.int64)                    # (m, nd)
    lin = (t * np.array(strides, dtype=np.int64)).sum(axis=1)
    idx = np.arange(n, dtype=np.int64)
    mask = np.ones((n, m), dtype=bool)
    rem = idx
    for k in range(nd):
        ck = rem // strides[k]
        rem = rem % strides[k]
        # valid[s] for shift s in (-1, 0, 1) of coordinate k
        valid = np.stack([ck >= 1, np.ones(n, dtype=bool), ck <= dims[k] - 2], axis=1)
        mask &= valid[:, t[:, k] + 1]
    cols = (idx.astype(np.int32)[:, None] + lin.astype(np.int32)[None, :])
    isdiag = lin == 0
    if noise != 0.0:
        gv = streams(seed)[1]
        vals = off + noise * gv.standard_normal((n, m))
    else:
        vals = np.full((n, m), off)
    vals[:, isdiag] = diag
    return _from_table(n, mask, cols, vals)


def stencil_nnz(m: int, ndim: int, kind: str) -> int:
    """Stored entries of a star/box stencil on an m^ndim grid (closed form)."""
    if kind == "star":
        return (2 * ndim + 1) * m ** ndim - 2 * ndim * m ** (ndim - 1)
    return (3 * m - 2) ** ndim


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------

def c1_laplace2d(m: int = 64) -> CSR:
    """2-D 5-point Laplacian, m x m grid, diag 4 and neighbours -1 (seed 1001)."""
    return stencil((m, m), "star", 4.0, -1.0)


def c3_stencil27(m: int = 128, noise: float = 1e-3, seed: int = 1003) -> CSR:
    """3-D 27-point stencil on m^3, diag 26, neighbours -1 + noise N(0,1)."""
    return stencil((m, m, m), "box", 26.0, -1.0, noise=noise, seed=seed)


def c2_hmep(n: int = 6_200_000, nbands: int = 14, dmax: int = 2_000_000,
            run: int = 15_000, gap: int = 10_000, seed: int = 1002) -> CSR:
    """Banded symmetric matrix shaped like HMEp.

    14 seeded offsets d_k in [1, dmax], each mirrored (+-d_k) so that the
    matrix is symmetric.  Band k holds the pair (i, i+d_k) / (i+d_k, i) when
    ``(i + phase_k) mod (run + gap) < run``: present in runs of ``run`` rows,
    absent in gaps of ``gap`` rows.  Values N(0,1); a mirrored pair shares its
    value; the diagonal is N(0,1) too.
    """
    gp, gv, _, _ = streams(seed)
    d = np.sort(gp.choice(np.arange(1, dmax + 1, dtype=np.int64), nbands, replace=False))
    phase = gp.integers(0, run + gap, nbands)
    diagv = gv.standard_normal(n)
    bandv = gv.standard_normal((nbands, n))
    i = np.arange(n, dtype=np.int64)[:, None]
    per = run + gap
    # upper entry (i, i + d_k) lives in row i; its mirror (r, r - d_k) in row r
    up = (i + d[None, :] < n) & (((i + phase[None, :]) % per) < run)
    src_row = i - d[::-1][None, :]                       # r - d_k, offsets ascending
    lo = (src_row >= 0) & (((src_row + phase[::-1][None, :]) % per) < run)
    mask = np.concatenate([lo, np.ones((n, 1), dtype=bool), up], axis=1)
    offs = np.concatenate([-d[::-1], [0], d]).astype(np.int32)
    cols = np.arange(n, dtype=np.int32)[:, None] + offs[None, :]
    kk = np.arange(nbands)[::-1]
    lov = bandv[kk[None, :], np.clip(src_row, 0, None)]
    vals = np.concatenate([lov, diagv[:, None], bandv.T], axis=1)
    return _from_table(n, mask, cols, vals)


def _dedupe_sorted(n: int, keys: np.ndarray, draw) -> np.ndarray:
    """Remove repeated keys of a sorted ``row * n + col`` array by redrawing.

    A repeated column in a row is replaced by a fresh ``draw(rows)`` candidate
    until every row holds distinct columns; the result stays sorted.
    """
    dup = np.zeros(keys.size, dtype=bool)
    dup[1:] = keys[1:] == keys[:-1]
    if not dup.any():
        return keys
    kept = keys[~dup]
    extra = np.empty(0, dtype=np.int64)     # accepted redraws, sorted
    pending = keys[dup] // n

    def member(sorted_keys, q):
        pos = np.searchsorted(sorted_keys, q)
        hit = pos < sorted_keys.size
        out = np.zeros(q.size, dtype=bool)
        out[hit] = sorted_keys[pos[hit]] == q[hit]
        return out

    while pending.size:
        new = pending * n + draw(pending)
        new.sort()
        bad = np.zeros(new.size, dtype=bool)
        bad[1:] = new[1:] == new[:-1]
        bad |= member(kept, new) | member(extra, new)
        extra = np.sort(np.concatenate([extra, new[~bad]]))
        pending = new[bad] // n
    return np.insert(kept, np.searchsorted(kept, extra), extra)


def _random_pattern(n: int, lens: np.ndarray, draw, seq: np.random.SeedSequence,
                    chunk: int = 1 << 24):
    """Columns for rows of the given lengths: distinct per row, ascending.

    Rows are cut into consecutive chunks of about ``chunk`` entries.  Chunk c
    draws with its own generator ``PCG64(seq.spawn(...)[c])``, so the result
    does not depend on how many threads run the chunks.  Each chunk draws
    ``draw(rows, g)`` for all its entries, sorts by (row, col) and redraws
    duplicates.  Returns (int64 rowptr, int32 columns in CSR order).
    """
    import concurrent.futures as cf
    import os
    rowptr = np.zeros(n + 1, dtype=np.int64)
    np.cumsum(lens, out=rowptr[1:])
    col = np.empty(int(rowptr[-1]), dtype=np.int32)
    bounds = [0]
    while bounds[-1] < n:
        r0 = bounds[-1]
        r1 = int(np.searchsorted(rowptr, rowptr[r0] + chunk, side="right")) - 1
        bounds.append(min(max(r1, r0 + 1), n))
    seqs = seq.spawn(len(bounds) - 1)

    def work(c):
        r0, r1 = bounds[c], bounds[c + 1]
        g = np.random.Generator(np.random.PCG64(seqs[c]))
        rows = np.repeat(np.arange(r0, r1, dtype=np.int64), lens[r0:r1])
        keys = rows * n + draw(rows, g)
        del rows
        keys.sort()
        keys = _dedupe_sorted(n, keys, lambda r: draw(r, g))
        col[rowptr[r0]:rowptr[r1]] = keys % n

    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with cf.ThreadPoolExecutor(workers) as ex:
        list(ex.map(work, range(len(bounds) - 1)))
    return rowptr, col


def c4_powerlaw(n: int = 4_000_000, mean: float = 10.0, sigma: float = 1.0,
                lmax: int = 50_000, nlong: int = 64, long_lo: int = 20_000,
                long_hi: int = 50_000, seed: int = 1004) -> CSR:
    """Irregular matrix with lognormal row lengths and a few very long rows.

    len_i = clip(rint(LogNormal(mu, sigma)), 1, lmax) with mu = ln(mean) -
    sigma^2/2 (so the unclipped mean is ``mean``); then ``nlong`` seeded rows
    get U{long_lo..long_hi}.  Columns uniform on [0, n) without duplicates in a
    row, sorted; values U[-1, 1).
    """
    gp, gv, _, _ = streams(seed)
    mu = np.log(mean) - sigma * sigma / 2.0
    lens = np.clip(np.rint(gp.lognormal(mu, sigma, n)), 1, lmax).astype(np.int64)
    longrows = gp.choice(n, nlong, replace=False)
    lens[longrows] = gp.integers(long_lo, long_hi + 1, nlong)
    rowptr, col = _random_pattern(n, lens, lambda r, g: g.integers(0, n, r.size),
                                  np.random.SeedSequence(seed).spawn(5)[4])
    val = gv.uniform(-1.0, 1.0, col.size)
    return CSR(n, rowptr, col, val)


def c5_fem(n: int = 8_000_000, lo: int = 20, hi: int = 40, frac_long: float = 0.01,
           long_len: int = 2000, band: int = 10_000, p_near: float = 0.95,
           seed: int = 1005) -> CSR:
    """FEM-like partition block: short rows plus 1% rows of 2,000 entries.

    len_i ~ U{lo..hi}; round(frac_long * n) seeded rows get ``long_len``.  Each
    column is drawn with probability p_near uniformly from
    [max(0, i-band), min(n-1, i+band)] and otherwise uniformly from [0, n);
    duplicates in a row are redrawn by the same rule; columns sorted; values
    N(0, 1).
    """
    gp, gv, _, _ = streams(seed)
    lens = gp.integers(lo, hi + 1, n).astype(np.int64)
    nlong = int(round(frac_long * n))
    longrows = gp.choice(n, nlong, replace=False)
    lens[longrows] = long_len
    def draw(rows, g):
        near = g.random(rows.size) < p_near
        a = np.maximum(rows - band, 0)
        w = np.minimum(rows + band, n - 1) + 1 - a
        c_near = a + (g.random(rows.size) * w).astype(np.int64)
        c_far = g.integers(0, n, rows.size)
        return np.where(near, c_near, c_far)

    rowptr, col = _random_pattern(n, lens, draw, np.random.SeedSequence(seed).spawn(5)[4])
    val = gv.standard_normal(col.size)
    return CSR(n, rowptr, col, val)


# --------------------------------------------------------------------------
# small random matrices for edge cases
# --------------------------------------------------------------------------

def random_csr(n: int, seed: int, density: float = 0.05, empty_frac: float = 0.0,
               long_rows: int = 0, long_len: int | None = None,
               dup_frac: float = 0.0, zero_frac: float = 0.0,
               unsorted: bool = False, dtype=np.float64,
               lens: np.ndarray | None = None) -> CSR:
    """A small random CSR matrix with optional awkward features.

    empty rows, very long rows, duplicated (row, col) entries, explicit zeros
    and unsorted columns are all legal input and are kept as stored entries.
    ``lens`` overrides the drawn row lengths.
    """
    gp, gv, _, _ = streams(seed)
    if lens is None:
        lam = max(density * n, 0.0)
        lens = gp.poisson(lam, n).astype(np.int64)
        if empty_frac > 0:
            lens[gp.random(n) < empty_frac] = 0
        if long_rows > 0 and n > 0:
            rows = gp.choice(n, min(long_rows, n), replace=False)
            lens[rows] = long_len if long_len is not None else n
    lens = np.asarray(lens, dtype=np.int64)
    rowptr = np.zeros(n + 1, dtype=np.int64)
    np.cumsum(lens, out=rowptr[1:])
    nnz = int(rowptr[-1])
    col = gp.integers(0, max(n, 1), nnz).astype(np.int64)
    if dup_frac > 0 and nnz > 1:
        # copy the previous entry's column inside the same row
        row_of = np.repeat(np.arange(n), lens)
        pick = np.nonzero(gp.random(nnz) < dup_frac)[0]
        pick = pick[pick > 0]
        pick = pick[row_of[pick] == row_of[pick - 1]]
        col[pick] = col[pick - 1]
    if not unsorted:
        for i in range(n):
            s, e = rowptr[i], rowptr[i + 1]
            col[s:e] = np.sort(col[s:e])
    val = gv.uniform(-1.0, 1.0, nnz)
    if zero_frac > 0 and nnz:
        val[gv.random(nnz) < zero_frac] = 0.0
    return CSR(n, rowptr, col.astype(np.int32), val.astype(dtype))


# --------------------------------------------------------------------------

WORKLOADS = {
    "c1_laplace2d_64": (c1_laplace2d, 1001),
    "c2_hmep_6.2m": (c2_hmep, 1002),
    "c3_stencil27_128": (c3_stencil27, 1003),
    "c4_powerlaw_4m": (c4_powerlaw, 1004),
    "c5_fem_8m": (c5_fem, 1005),
}


def by_name(name: str, dtype=np.float64):
    """(matrix, x, y0, seed) for a named workload; fp32 values rounded from fp64."""
    fn, seed = WORKLOADS[name]
    a = fn()
    x, y0 = vectors(a.n, seed, np.float64)
    if dtype == np.float32:
        a = as_fp32(a)
        x = x.astype(np.float32)
        y0 = y0.astype(np.float32)
    return a, x, y0, seed
