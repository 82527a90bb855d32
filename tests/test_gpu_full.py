"""GPU parity at the five workloads' full sizes, in the launch configuration the
benchmark times: every format is built from the full matrix, applied to the
full vector and checked against the oracle on every row.  ELL-R of the
power-law matrix (~2.4 TB padded) must be refused with FOOTPRINT.  The layouts
the device converters build at full size (64-bit slot offsets, grid-stride
fills, ragged last blocks, the device-built chunk lists' slices) are compared
byte for byte with the oracle's converters."""
import sys
import time

import numpy as np
import pytest
import torch

import gen
import oracle

from gpu_util import FORMATS, TOL, apply, to_dev

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import sparse_formats_amd as sf

CASES = [
    ("c1_laplace2d_64", torch.float64),
    ("c2_hmep_6.2m", torch.float64),
    ("c3_stencil27_128", torch.float64),
    ("c3_stencil27_128", torch.float32),
    ("c4_powerlaw_4m", torch.float64),
    ("c5_fem_8m", torch.float64),
]
AB = [(1.0, 0.0), (-1.5, 0.5)]
# besides each format's automatic choice: the CSR column-slice kernel, SELL-64
# with and without the LDS window and the HYB/HEC tail kernels where those are
# candidates
EXTRA = {
    "c4_powerlaw_4m": [("csr", dict(csr_kernel="xblock")), ("csr", dict(csr_kernel="balanced"))],
    "c5_fem_8m": [("sell64", dict(x_window=0)), ("sell64", dict(x_window=1)),
                  ("csr", dict(csr_kernel="vector")), ("hec", dict(csr_kernel="xblock")),
                  ("hec", dict(csr_kernel="balanced")), ("hyb", dict(csr_kernel="xblock")),
                  ("hyb", dict(csr_kernel="balanced"))],
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.mark.parametrize("name,dtype", CASES, ids=["%s-%s" % (n, str(d)[6:]) for n, d in CASES])
def test_full_size(name, dtype):
    t0 = time.time()
    npdt = np.float64 if dtype == torch.float64 else np.float32
    a, x_np, y0_np, _ = gen.by_name(name, npdt)
    log("[full] %s %s: n=%d nnz=%d generated in %.1fs" % (name, dtype, a.n, a.nnz,
                                                           time.time() - t0))
    t0 = time.time()
    refs = {ab: oracle.spmv(a, x_np, y0_np, ab[0], ab[1], nthreads=0) for ab in AB}
    log("[full]   oracle on every row in %.1fs" % (time.time() - t0))
    M = sf.Matrix.from_csr(*to_dev(a, dtype), n=a.n)
    torch.cuda.empty_cache()
    x = torch.from_numpy(x_np).cuda()
    y0 = torch.from_numpy(y0_np).cuda()
    for fmt, kw in [(f, {}) for f in FORMATS] + EXTRA.get(name, []):
        try:
            M.convert(fmt, **kw)
        except sf.SpmvError as e:
            assert name.startswith("c4") and fmt == "ellr" and e.code == -4, str(e)
            log("[full]   %s refused: %s" % (fmt, e))
            continue
        assert not (name.startswith("c4") and fmt == "ellr"), "ELL-R of C4 must be refused"
        for alpha, beta in AB:
            y = apply(M, x, y0, alpha, beta)
            ref, scale = refs[(alpha, beta)]
            ok, worst, k = oracle.check(y, ref, scale, TOL[dtype])
            assert ok, "%s %s %s a=%g b=%g: row %d err/tol %.3g (gpu %r ref %r)" % (
                name, fmt, kw, alpha, beta, k, worst, float(y[k]), float(ref[k]))
        log("[full]   %s %s ok on all %d rows (worst err/tol %.3g) %s"
            % (fmt, kw, a.n, worst, M.info()))
    M.close()
    torch.cuda.empty_cache()


def _same_ell(M, oc, ov, ol):
    assert np.array_equal(M.export("ell_col"), oc)
    assert M.export("ell_val").tobytes() == ov.tobytes()
    assert np.array_equal(M.export("ell_len"), ol)


def _same_sell(M, a, sigma):
    perm, sp, ls, sc, sv = oracle.sell(a, sigma=sigma)
    assert np.array_equal(M.export("sell_perm"), perm.astype(np.int32))
    assert np.array_equal(M.export("sell_slice_ptr"), sp)
    assert np.array_equal(M.export("sell_len"), ls)
    assert np.array_equal(M.export("sell_col"), sc)
    assert M.export("sell_val").tobytes() == sv.tobytes()


def _same_split(M, a, fmt):
    i = M.info()
    K, sigma = i["ell_width"], i["sort_window"]
    assert K in (oracle.hyb_width(a), max(oracle.hyb_width(a), oracle.regular_width(a)))
    assert sigma == (oracle.ELL_BLOCK_SPLIT if oracle.ell_pad_fraction(a, K) > 0.1 else 0)
    oc, ov, ol, op = oracle.ell(a, K, block=oracle.ELL_BLOCK_SPLIT, sigma=sigma, with_perm=True)
    _same_ell(M, oc, ov, ol)
    del oc, ov
    if sigma > 0:
        assert np.array_equal(M.export("ell_perm"), op.astype(np.int32))
    trow, tptr, tcol, tval = oracle.tail(a, K)
    assert i["tail_nnz"] == tcol.size
    if fmt == "hyb":
        assert np.array_equal(M.export("tail_row"), trow)
    else:
        assert np.array_equal(M.export("tail_ptr"), tptr)
    assert np.array_equal(M.export("tail_col"), tcol)
    assert M.export("tail_val").tobytes() == tval.tobytes()
    return K, sigma


@pytest.mark.parametrize("name", ["c3_stencil27_128", "c5_fem_8m"])
def test_full_size_layouts(name):
    """Byte-exact layouts at full size: the 27-point stencil in every format;
    the FEM block in SELL-64 (8,192-row sort windows, and 1,024 with the LDS
    window), HYB and HEC.  ELL-R of the FEM block is 197 GB, more than the
    host holds for the comparison: only its slot count and footprint are
    checked (its values are covered by the every-row product test)."""
    t0 = time.time()
    a, _, _, _ = gen.by_name(name)
    M = sf.Matrix.from_csr(*to_dev(a), n=a.n)
    assert np.array_equal(M.export("rowptr"), a.rowptr.astype(np.int32))
    assert np.array_equal(M.export("col"), a.col)
    assert M.export("val").tobytes() == a.val.tobytes()
    M.convert("ellr")
    S, W = -(-a.n // 64) * 64, int(a.row_lengths().max())
    assert M.info()["slots"] == S * W and M.info()["ell_stride"] == S
    if name.startswith("c3"):
        _same_ell(M, *oracle.ell(a))
    M.convert("sell64", x_window=0)
    _same_sell(M, a, 8192)
    M.convert("sell64", x_window=1)
    _same_sell(M, a, 1024)
    for fmt in ("hyb", "hec"):
        M.convert(fmt)
        K, sigma = _same_split(M, a, fmt)
        log("[layout] %s %s K=%d sort_window=%d matches" % (name, fmt, K, sigma))
    M.close()
    torch.cuda.empty_cache()
    log("[layout] %s done in %.1fs" % (name, time.time() - t0))
