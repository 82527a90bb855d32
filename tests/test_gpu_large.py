"""Row counts large enough that the grids of the per-row kernels would pass
HIP's 2^32 work-item limit (a group of S lanes per row, G wave groups per
64-row tile): launches are split, and every format still matches the oracle.
The largest case is the largest n the library takes, 2^31 - 2 (row and column
indices up to 2^31 - 3, padded row counts of 2^31); the column-slice CSR
kernel, which counts the entries of every row in each of its 9 tiles (8
column slices and the row range's band; 9 n counts), is refused there and run
at the most rows it takes.

The matrix has n rows (300,000,000, then 2^31 - 2), at most three entries in
a row, and its
entries in a few hundred rows spread over the whole range (columns up to
n - 1).  It is built from COO triples on the device; x is drawn on the device
and only the entries the matrix reads are copied back, so the oracle runs on
the touched rows alone (a compact CSR over the columns used) and every other
row must come out as exactly beta * y0."""
import numpy as np
import pytest
import torch

import oracle
from gen import CSR

from gpu_util import TOL

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import sparse_formats_amd as sf

SIZES = [300_000_000, 2 ** 31 - 2]


def _triples(N, seed=101):
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([
        [0, 1, 2, 63, 64, 65, N // 2, N - 65, N - 64, N - 2, N - 1],
        rng.integers(0, N, 400)])).astype(np.int64)
    lens = rng.integers(1, 4, rows.size)
    r = np.repeat(rows, lens)
    c = rng.integers(0, N, r.size).astype(np.int64)
    c[::7] = N - 1
    c[1::11] = 0
    c[2::13] = r[2::13]                       # some diagonal entries
    v = rng.standard_normal(r.size)
    return r, c.astype(np.int32), v


# the most rows the column-slice CSR kernel takes (9 n counts below 2^31 - 16)
XB_MAX = (2 ** 31 - 1 - 16) // 9


@pytest.fixture(scope="module", params=SIZES, ids=["300M", "2^31-2"])
def large(request):
    yield from _large(request.param)


@pytest.fixture(scope="module")
def xb_largest():
    yield from _large(XB_MAX)


def _large(N):
    r, c, v = _triples(N)
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    x = torch.rand(N, dtype=torch.float64, device="cuda", generator=g) * 2 - 1
    M = sf.Matrix.from_coo(torch.from_numpy(r).cuda(), torch.from_numpy(c).cuda(),
                           torch.from_numpy(v).cuda(), n=N)
    # compact reference: the touched rows, columns renumbered into x_used
    used = np.unique(c)
    x_used = x[torch.from_numpy(used.astype(np.int64)).cuda()].cpu().numpy()
    order = np.lexsort((np.arange(r.size), r))          # by row, then input order
    rs, cs, vs = r[order], c[order], v[order]
    rows, counts = np.unique(rs, return_counts=True)
    rp = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    compact = CSR(rows.size, rp, np.searchsorted(used, cs).astype(np.int32), vs)
    yield N, M, x, rows, compact, x_used
    M.close()
    del x
    torch.cuda.empty_cache()


def _check(N, M, x, rows, compact, x_used, what):
    alpha, beta = 1.5, 0.5
    y = torch.full((N,), 2.0, dtype=torch.float64, device="cuda")
    M.apply(y, x, alpha, beta)
    torch.cuda.synchronize()
    touched = torch.from_numpy(rows).cuda()
    got = y[touched].cpu().numpy()
    ref, scale = oracle.spmv(compact, x_used, np.full(rows.size, 2.0), alpha, beta)
    ok, worst, k = oracle.check(got, ref, scale, TOL[torch.float64])
    assert ok, "%s: worst %.3g at row %d" % (what, worst, rows[k])
    y[touched] = 1.0
    assert int((y != 1.0).sum()) == 0, what   # untouched rows: beta * y0 = 1 exactly


@pytest.mark.parametrize("fmt,kw", [
    ("csr", dict(csr_kernel="vector", subwave=64, csr_rows=1, csr_stage=0)),
    ("csr", dict(csr_kernel="vector", subwave=16, csr_rows=1, csr_stage=1)),
    ("csr", dict(csr_kernel="balanced")),
    ("ellr", dict(ell_groups=16)),
    ("ellr", dict(ell_groups=1)),
    ("sell64", {}),
    ("hyb", {}),
    ("hec", {}),
    ("csr", dict(csr_kernel="xblock")),
])
def test_many_rows(large, fmt, kw):
    N, M, x, rows, compact, x_used = large
    if kw.get("csr_kernel") == "xblock":
        # 9 n counts would pass 2^31: refused, handle kept
        with pytest.raises(sf.SpmvError) as e:
            M.convert(fmt, **kw)
        assert e.value.code == -1
        M.convert("csr", csr_kernel="balanced")
        _check(N, M, x, rows, compact, x_used, "n=%d after a refused xblock" % N)
        return
    if fmt == "ellr" and N > 2 ** 30:
        # 3 x 2^31 slots (77 GB) exceed a 1 GiB budget: refused, handle kept
        with pytest.raises(sf.SpmvError) as e:
            M.convert(fmt, footprint_budget=1 << 30, **kw)
        assert e.value.code == -4
        return
    M.convert(fmt, **kw)
    _check(N, M, x, rows, compact, x_used, "n=%d %s %s" % (N, fmt, kw))


def test_xblock_most_rows(xb_largest):
    """The column-slice CSR kernel at the most rows it takes: 9 n counts up
    to 2^31 - 17, about 11,600 row ranges of at most 20,480 rows."""
    N, M, x, rows, compact, x_used = xb_largest
    M.convert("csr", csr_kernel="xblock")
    assert M.info()["csr_kernel"] == "xblock"
    _check(N, M, x, rows, compact, x_used, "n=%d xblock" % N)


# -- the largest entry count the library takes ---------------------------------

NNZ_MAX = 2 ** 31 - 65537
N_WIDE = 100_000_000


@pytest.fixture(scope="module")
def many_entries():
    """n = 10^8 rows of 21 or 22 entries, nnz = 2^31 - 65537 exactly, built on
    the device (random columns, N(0,1) values); the oracle checks sampled rows."""
    n = N_WIDE
    extra = NNZ_MAX - 21 * n
    lens = torch.full((n,), 21, dtype=torch.int64, device="cuda")
    lens[:extra] += 1
    rowptr = torch.zeros(n + 1, dtype=torch.int64, device="cuda")
    rowptr[1:] = torch.cumsum(lens, 0)
    del lens
    assert int(rowptr[-1]) == NNZ_MAX
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    col = torch.randint(0, n, (NNZ_MAX,), dtype=torch.int32, device="cuda", generator=g)
    val = torch.randn(NNZ_MAX, dtype=torch.float64, device="cuda", generator=g)
    x = torch.rand(n, dtype=torch.float64, device="cuda", generator=g) * 2 - 1
    M = sf.Matrix.from_csr(rowptr, col, val, n=n)
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, 1, extra - 1, extra, n // 2, n - 2, n - 1],
                                     rng.integers(0, n, 3000)])).astype(np.int64)
    rp = rowptr.cpu().numpy()
    idx = np.concatenate([np.arange(rp[r], rp[r + 1]) for r in rows])
    idx_t = torch.from_numpy(idx).cuda()
    cs = col[idx_t].cpu().numpy()
    vs = val[idx_t].cpu().numpy()
    used = np.unique(cs)
    x_used = x[torch.from_numpy(used.astype(np.int64)).cuda()].cpu().numpy()
    lens_s = (rp[rows + 1] - rp[rows]).astype(np.int64)
    crp = np.concatenate([[0], np.cumsum(lens_s)]).astype(np.int64)
    compact = CSR(rows.size, crp, np.searchsorted(used, cs).astype(np.int32), vs)
    del rowptr, col, val, idx_t
    torch.cuda.empty_cache()
    yield n, M, x, rows, compact, x_used
    M.close()
    del x
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt,kw", [
    ("csr", dict(csr_kernel="vector", subwave=16, csr_rows=1, csr_stage=1)),
    ("csr", dict(csr_kernel="vector", subwave=16, csr_rows=2, csr_stage=0)),
    ("csr", dict(csr_kernel="balanced")),
    ("ellr", {}),
    ("sell64", {}),
    ("hyb", dict(ell_width=10)),
    ("hec", dict(ell_width=10)),
    ("csr", dict(csr_kernel="xblock")),
])
def test_most_entries(many_entries, fmt, kw):
    n, M, x, rows, compact, x_used = many_entries
    M.convert(fmt, **kw)
    alpha, beta = -0.75, 0.5
    y = torch.full((n,), 2.0, dtype=torch.float64, device="cuda")
    M.apply(y, x, alpha, beta)
    torch.cuda.synchronize()
    got = y[torch.from_numpy(rows).cuda()].cpu().numpy()
    ref, scale = oracle.spmv(compact, x_used, np.full(rows.size, 2.0), alpha, beta)
    ok, worst, k = oracle.check(got, ref, scale, TOL[torch.float64])
    assert ok, "nnz=%d %s %s: worst %.3g at row %d" % (NNZ_MAX, fmt, kw, worst, rows[k])
