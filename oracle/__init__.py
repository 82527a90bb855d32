"""CPU oracle for SpMV and the storage-format conversions -- test infrastructure.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package.  The GPU library never does; the two share no code.  The
arithmetic lives in ``oracle.c`` (plain C, built with gcc); this module only
marshals numpy arrays into it and states the tolerance test.

Functions (each restates a definition from the pages; see oracle.c):

* ``spmv``       -- y = alpha*A*x + beta*y with Dot2 row sums in fp64, and
                    the per-row scale |alpha|*sum|a*x| + |beta*y|.
* ``ell``        -- ELLPACK arrays: ELLPACK-R (column-major, stride a multiple of
                    64) or the HYB/HEC ELL part (column-major blocks of rows).
* ``sell``       -- SELL-64 (sorted, sliced, padded) arrays and permutation,
                    optionally sorted only inside windows of sigma rows.
* ``ell_pad_fraction`` -- share of padding slots a lane-per-row sweep of an
                    unsorted ELL part reads (the windowed-sort decision).
* ``hyb_width``  -- the ELL width of the HYB/HEC split (the ceil(n/3) rule).
* ``regular_width`` -- the other width candidate (99 % of rows fit whole).
* ``tail``       -- the irregular part of the split as COO and CSR.
* ``check``      -- the per-entry tolerance test |y - y_ref| <= tol * scale.
* ``cg``, ``bicgstab`` -- textbook Krylov solvers over the product (fp64).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB names a library built from a modified copy of oracle.c: the
# tests that check that the pins catch planted mistakes run the pin suite
# against it.  It is loaded as it is, never rebuilt.
_PLANTED = os.environ.get("ORACLE_LIB")
_SO = _PLANTED or os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.c")
_lib = None

TOL_F64 = 1e-12
TOL_F32 = 1e-5


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math, no FMA contraction)."""
    if _PLANTED:
        return _SO
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=False)
        lib = ctypes.CDLL(_SO)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.oracle_spmv.argtypes = [I64, P, P, P, P, P, ctypes.c_double, ctypes.c_double,
                                    P, P, P, I64, ctypes.c_int]
        lib.oracle_spmv.restype = ctypes.c_int
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_max_len.argtypes = [I64, P]
        lib.oracle_max_len.restype = I64
        lib.oracle_ell.argtypes = [I64, P, P, P, ctypes.c_int, I64, I64, I64, P, P, P, P]
        lib.oracle_ell_pad_fraction.argtypes = [I64, P, I64]
        lib.oracle_ell_pad_fraction.restype = ctypes.c_double
        lib.oracle_sell_layout.argtypes = [I64, P, I64, P, P, P]
        lib.oracle_sell_layout.restype = I64
        lib.oracle_sell_fill.argtypes = [I64, P, P, P, ctypes.c_int, P, P, ctypes.c_int, P, P]
        lib.oracle_hyb_width.argtypes = [I64, P, I64]
        lib.oracle_hyb_width.restype = I64
        lib.oracle_regular_width.argtypes = [I64, P]
        lib.oracle_regular_width.restype = I64
        lib.oracle_tail_nnz.argtypes = [I64, P, I64]
        lib.oracle_tail_nnz.restype = I64
        lib.oracle_tail.argtypes = [I64, P, P, P, ctypes.c_int, I64, P, P, P, P]
        for f in (lib.oracle_cg, lib.oracle_bicgstab):
            f.argtypes = [I64, P, P, P, P, P, ctypes.c_double, ctypes.c_int, P]
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def spmv(a, x, y0=None, alpha: float = 1.0, beta: float = 0.0, rows=None,
         nthreads: int = 1):
    """(y_ref, scale) in fp64 for y = alpha*A*x + beta*y0.

    fp32 values and vectors are promoted to fp64 exactly.  ``rows`` restricts
    the computation to the listed rows (outputs follow the list order).
    """
    lib = _load()
    rowptr = _c(a.rowptr, np.int64)
    col = _c(a.col, np.int32)
    val = _c(a.val, np.float64)
    xx = _c(x, np.float64)
    yy = None if (beta == 0.0 or y0 is None) else _c(y0, np.float64)
    if beta != 0.0 and yy is None:
        raise ValueError("beta != 0 needs y0")
    rr = None if rows is None else _c(rows, np.int64)
    m = a.n if rr is None else rr.size
    y = np.empty(m, dtype=np.float64)
    sc = np.empty(m, dtype=np.float64)
    lib.oracle_spmv(a.n, _p(rowptr), _p(col), _p(val), _p(xx), _p(yy),
                    float(alpha), float(beta), _p(y), _p(sc), _p(rr),
                    0 if rr is None else rr.size, int(nthreads))
    return y, sc


def check(y, y_ref, scale, tol: float):
    """Max over rows of |y - y_ref| / scale; rows with scale 0 must match exactly.

    Returns (ok, worst_ratio, worst_row).
    """
    y = np.asarray(y, dtype=np.float64)
    diff = np.abs(y - y_ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(scale > 0, diff / np.where(scale > 0, scale, 1.0),
                         np.where(diff == 0, 0.0, np.inf))
    ratio = np.where(np.isnan(ratio), np.inf, ratio)
    if ratio.size == 0:
        return True, 0.0, -1
    k = int(np.argmax(ratio))
    worst = float(ratio[k])
    return worst <= tol, worst / tol if tol > 0 else worst, k


def pad64(n: int) -> int:
    return (n + 63) // 64 * 64


def max_len(a) -> int:
    return int(_load().oracle_max_len(a.n, _p(_c(a.rowptr, np.int64))))


ELL_BLOCK_SPLIT = 1024   # rows per column-major block of the HYB/HEC ELL part


def ell(a, width: int | None = None, block: int = 0, sigma: int = 0, with_perm: bool = False):
    """ELLPACK arrays of the given width (default: longest row).

    block == 0: ELLPACK-R, one column-major block of pad64(n) rows.
    block > 0: column-major blocks of `block` rows (the HYB/HEC ELL part);
    sigma > 0 (dividing block) orders the rows of each aligned window of
    sigma positions by stored length descending, then row ascending.
    Returns (col[W*R] int32, val[W*R], len[R] int32[, perm[R] int64]), R the
    padded rows, lengths and perm by position.
    """
    lib = _load()
    rowptr = _c(a.rowptr, np.int64)
    W = max_len(a) if width is None else int(width)
    R = pad64(a.n) if block <= 0 else -(-a.n // block) * block
    val = np.ascontiguousarray(a.val)
    oc = np.empty(W * R, dtype=np.int32)
    ov = np.empty(W * R, dtype=val.dtype)
    ol = np.empty(R, dtype=np.int32)
    op = np.empty(R, dtype=np.int64)
    lib.oracle_ell(a.n, _p(rowptr), _p(_c(a.col, np.int32)), _p(val), val.itemsize,
                   W, int(block), int(sigma), _p(oc), _p(ov), _p(ol), _p(op))
    return (oc, ov, ol, op) if with_perm else (oc, ov, ol)


def ell_pad_fraction(a, width: int) -> float:
    """Share of the slots a lane-per-row sweep of the unsorted ELL part reads
    past the rows' ends (waves of 64 consecutive rows run to their longest)."""
    return float(_load().oracle_ell_pad_fraction(a.n, _p(_c(a.rowptr, np.int64)), int(width)))


def sell(a, sigma: int = 0, permuted: bool = False):
    """SELL-64: (perm[n] int64, slice_ptr[S/64+1] int64, len_sorted[S] int32,
    col[slots] int32, val[slots]).  sigma > 0 sorts only inside aligned
    windows of sigma rows (0: all rows at once).  permuted: the columns of the
    permuted basis P A P^T ((P v)[r] = v[perm[r]])."""
    lib = _load()
    rowptr = _c(a.rowptr, np.int64)
    S = pad64(a.n)
    perm = np.empty(a.n, dtype=np.int64)
    sp = np.empty(S // 64 + 1, dtype=np.int64)
    ls = np.empty(S, dtype=np.int32)
    total = lib.oracle_sell_layout(a.n, _p(rowptr), int(sigma), _p(perm), _p(sp), _p(ls))
    val = np.ascontiguousarray(a.val)
    oc = np.empty(total, dtype=np.int32)
    ov = np.empty(total, dtype=val.dtype)
    lib.oracle_sell_fill(a.n, _p(rowptr), _p(_c(a.col, np.int32)), _p(val), val.itemsize,
                         _p(perm), _p(sp), int(bool(permuted)), _p(oc), _p(ov))
    return perm, sp, ls, oc, ov


def hyb_width(a, requested: int = -1) -> int:
    return int(_load().oracle_hyb_width(a.n, _p(_c(a.rowptr, np.int64)), int(requested)))


def regular_width(a) -> int:
    """The second HYB/HEC width candidate: the smallest k with at most 1 % of
    the rows longer than k."""
    return int(_load().oracle_regular_width(a.n, _p(_c(a.rowptr, np.int64))))


def tail(a, K: int):
    """Tail of the width-K split: (row[t] int32, ptr[n+1] int32, col[t] int32, val[t])."""
    lib = _load()
    rowptr = _c(a.rowptr, np.int64)
    t = int(lib.oracle_tail_nnz(a.n, _p(rowptr), int(K)))
    val = np.ascontiguousarray(a.val)
    orow = np.empty(t, dtype=np.int32)
    optr = np.empty(a.n + 1, dtype=np.int32)
    oc = np.empty(t, dtype=np.int32)
    ov = np.empty(t, dtype=val.dtype)
    lib.oracle_tail(a.n, _p(rowptr), _p(_c(a.col, np.int32)), _p(val), val.itemsize, int(K),
                    _p(orow), _p(optr), _p(oc), _p(ov))
    return orow, optr, oc, ov


def _solve(fn, a, b, x0, rtol, max_iter):
    rowptr = _c(a.rowptr, np.int64)
    val = _c(a.val, np.float64)
    bb = _c(b, np.float64)
    x = np.array(np.zeros(a.n) if x0 is None else x0, dtype=np.float64)
    rel = ctypes.c_double()
    it = fn(a.n, _p(rowptr), _p(_c(a.col, np.int32)), _p(val), _p(bb), _p(x), float(rtol),
            int(max_iter), ctypes.byref(rel))
    return x, int(it), rel.value


def cg(a, b, x0=None, rtol: float = 1e-10, max_iter: int = 1000):
    """Conjugate gradients (A symmetric positive definite): (x, iterations,
    ||r|| / ||b|| of the recurred residual)."""
    return _solve(_load().oracle_cg, a, b, x0, rtol, max_iter)


def bicgstab(a, b, x0=None, rtol: float = 1e-10, max_iter: int = 1000):
    """BiCGSTAB (general A): (x, iterations, ||r|| / ||b||)."""
    return _solve(_load().oracle_bicgstab, a, b, x0, rtol, max_iter)
