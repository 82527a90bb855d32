"""GPU parity on small and medium matrices: every format, both dtypes, several
alpha/beta, edge cases (empty rows, duplicates, explicit zeros, unsorted
columns, very long rows, n % 64 != 0, n = 1, nnz = 0), converter layouts
bit-exact against the oracle's reference converters, and the error paths."""
import numpy as np
import pytest
import torch

import oracle
from gen import CSR, c1_laplace2d, random_csr, stencil, vectors

from gpu_util import AB, FORMATS, TOL, apply, check, to_dev

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import sparse_formats_amd as sf


def _mats():
    return {
        "c1": lambda: c1_laplace2d(),
        "ragged": lambda: random_csr(3001, seed=41, density=0.003, empty_frac=0.25,
                                     long_rows=3, long_len=2500),
        "dups_unsorted": lambda: random_csr(777, seed=42, density=0.01, dup_frac=0.3,
                                            zero_frac=0.1, unsorted=True),
        "n1": lambda: CSR(1, np.array([0, 3], np.int64), np.array([0, 0, 0], np.int32),
                          np.array([1.0, -2.0, 0.5])),
        "nnz0": lambda: CSR(130, np.zeros(131, np.int64), np.zeros(0, np.int32), np.zeros(0)),
        "n0": lambda: CSR(0, np.zeros(1, np.int64), np.zeros(0, np.int32), np.zeros(0)),
        "box27": lambda: stencil((13, 11, 9), "box", 26.0, -1.0, noise=1e-3, seed=3),
        "every_len": lambda: random_csr(700, seed=43, lens=np.arange(700) % 601),
        "long_spans": lambda: random_csr(5000, seed=44, lens=np.where(
            np.arange(5000) % 997 == 0, 4000, np.arange(5000) % 7)),
    }


MATS = _mats()


@pytest.mark.parametrize("dtype", [torch.float64, torch.float32])
@pytest.mark.parametrize("name", list(MATS))
@pytest.mark.parametrize("fmt", FORMATS)
def test_format_parity(fmt, name, dtype):
    a = MATS[name]()
    if dtype == torch.float32:
        a = CSR(a.n, a.rowptr, a.col, a.val.astype(np.float32))
    x_np, y0_np = vectors(a.n, 7)
    npdt = np.float64 if dtype == torch.float64 else np.float32
    x_np, y0_np = x_np.astype(npdt), y0_np.astype(npdt)
    M = sf.Matrix.from_csr(*to_dev(a, dtype), n=a.n)
    M.convert(fmt)
    x = torch.from_numpy(x_np).cuda()
    y0 = torch.from_numpy(y0_np).cuda()
    for alpha, beta in AB:
        y = apply(M, x, y0, alpha, beta)
        check(a, x_np, y0_np, alpha, beta, y, dtype, what="%s/%s/%s a=%g b=%g" % (
            fmt, name, dtype, alpha, beta))
    M.close()


@pytest.mark.parametrize("fmt", ["hyb", "hec"])
@pytest.mark.parametrize("K", [0, 1, 5, 20, 10 ** 6])
def test_split_width_any(fmt, K):
    a = MATS["long_spans"]()
    x_np, y0_np = vectors(a.n, 8)
    M = sf.Matrix.from_csr(*to_dev(a), n=a.n).convert(fmt, ell_width=K)
    info = M.info()
    assert info["ell_width"] == min(K, oracle.max_len(a))
    x = torch.from_numpy(x_np).cuda()
    y0 = torch.from_numpy(y0_np).cuda()
    for alpha, beta in AB[:2]:
        check(a, x_np, y0_np, alpha, beta, apply(M, x, y0, alpha, beta), torch.float64,
              what="%s K=%d" % (fmt, K))


@pytest.mark.parametrize("rows", [1, 2, 4])
@pytest.mark.parametrize("sw", [1, 2, 4, 8, 16, 32, 64])
@pytest.mark.parametrize("name", ["every_len", "ragged", "nnz0", "n1", "c1"])
def test_csr_every_shape(sw, rows, name):
    a = MATS[name]()
    x_np, y0_np = vectors(a.n, 9)
    M = sf.Matrix.from_csr(*to_dev(a), n=a.n).convert("csr", subwave=sw, csr_rows=rows)
    assert M.info()["subwave"] == sw and M.info()["csr_rows"] == rows
    x = torch.from_numpy(x_np).cuda()
    y0 = torch.from_numpy(y0_np).cuda()
    for alpha, beta in AB[:2]:
        check(a, x_np, y0_np, alpha, beta, apply(M, x, y0, alpha, beta), torch.float64,
              what="csr S=%d R=%d %s" % (sw, rows, name))
    with pytest.raises(sf.SpmvError):
        M.convert("csr", csr_rows=3)
    with pytest.raises(sf.SpmvError):
        M.convert("csr", csr_rows=8)


@pytest.mark.parametrize("dtype", [torch.float64, torch.float32])
@pytest.mark.parametrize("sw", [2, 4, 8, 16])
@pytest.mark.parametrize("name", ["short", "every_len", "ragged", "dups_unsorted", "nnz0", "n1",
                                  "c1", "box27"])
def test_csr_staged(sw, name, dtype):
    """The LDS-staged vector kernel against the oracle, and bit for bit against
    the direct kernel of the same shape (same per-lane order).  "every_len"
    and "ragged" have waves too long for the slice, which read directly."""
    if name == "short":
        a = random_csr(20011, seed=45, lens=(np.arange(20011) * 7919) % 41)
    else:
        a = MATS[name]()
    npdt = np.float64 if dtype == torch.float64 else np.float32
    if dtype == torch.float32:
        a = CSR(a.n, a.rowptr, a.col, a.val.astype(np.float32))
    x_np, y0_np = (v.astype(npdt) for v in vectors(a.n, 19))
    x = torch.from_numpy(x_np).cuda()
    y0 = torch.from_numpy(y0_np).cuda()
    M = sf.Matrix.from_csr(*to_dev(a, dtype), n=a.n)
    M.convert("csr", csr_kernel="vector", subwave=sw, csr_rows=1, csr_stage=1)
    inf = M.info()
    assert inf["csr_stage_slots"] >= 256 and inf["subwave"] == sw and inf["csr_kernel"] == "vector"
    ys = []
    for alpha, beta in AB:
        y = apply(M, x, y0, alpha, beta)
        check(a, x_np, y0_np, alpha, beta, y, dtype, what="csr staged S=%d %s a=%g b=%g" % (
            sw, name, alpha, beta))
        ys.append(y)
    M.convert("csr", csr_kernel="vector", subwave=sw, csr_rows=1, csr_stage=0)
    assert M.info()["csr_stage_slots"] == 0
    for (alpha, beta), y_st in zip(AB, ys):
        assert np.array_equal(apply(M, x, y0, alpha, beta), y_st), (sw, name, alpha, beta)
    M.close()


@pytest.mark.parametrize("dtype", [torch.float64, torch.float32])
@pytest.mark.parametrize("name", ["c1", "ragged", "every_len", "long_spans", "box27", "nnz0",
                                  "dups_unsorted", "n1"])
@pytest.mark.parametrize("kernel", ["vector", "balanced", "xblock", "auto"])
@pytest.mark.parametrize("fmt", ["hec", "hyb"])
def test_tail_kernels(fmt, kernel, name, dtype):
    """HEC and HYB with each tail kernel (HEC: the vector and balanced CSR
    kernels; HYB: the balanced COO kernel, the vector kernel being no HYB
    tail kernel; both: the column-slice kernel adding onto the ELL part's y)
    and the timed choice against the oracle, at the default split and at K =
    1 (almost everything in the tail)."""
    a = MATS[name]()
    npdt = np.float64 if dtype == torch.float64 else np.float32
    if dtype == torch.float32:
        a = CSR(a.n, a.rowptr, a.col, a.val.astype(np.float32))
    x_np, y0_np = (v.astype(npdt) for v in vectors(a.n, 23))
    x = torch.from_numpy(x_np).cuda()
    y0 = torch.from_numpy(y0_np).cuda()
    M = sf.Matrix.from_csr(*to_dev(a, dtype), n=a.n)
    want = "balanced" if fmt == "hyb" and kernel == "vector" else kernel
    for K in (-1, 1):
        M.convert(fmt, ell_width=K, csr_kernel=kernel)
        inf = M.info()
        if inf["tail_nnz"] > 0 and kernel != "auto":
            assert inf["tail_kernel"] == want
        for alpha, beta in AB:
            check(a, x_np, y0_np, alpha, beta, apply(M, x, y0, alpha, beta), dtype,
                  what="%s tail %s K=%d %s a=%g b=%g" % (fmt, kernel, K, name, alpha, beta))
    M.close()


@pytest.mark.parametrize("dtype", [torch.float64, torch.float32])
@pytest.mark.parametrize("fmt,kw", [("ellr", {}), ("ellr", dict(ell_groups=4)),
                                    ("ellr", dict(x_window=1)), ("sell64", {}),
                                    ("hyb", dict(x_window=0)), ("hyb", dict(x_window=1)),
                                    ("hec", dict(csr_kernel="balanced")),
                                    ("csr", dict(csr_kernel="vector", csr_stage=1))])
@pytest.mark.parametrize("cache", [0, 1])
def test_col_cache_policies(fmt, kw, cache, dtype):
    """Column indices streamed (0) or cached (1): same results, both reported."""
    a = _banded() if kw.get("x_window") == 1 else MATS["long_spans"]()
    npdt = np.float64 if dtype == torch.float64 else np.float32
    if dtype == torch.float32:
        a = CSR(a.n, a.rowptr, a.col, a.val.astype(np.float32))
    x_np, y0_np = (v.astype(npdt) for v in vectors(a.n, 91))
    M = sf.Matrix.from_csr(*to_dev(a, dtype), n=a.n).convert(fmt, col_cache=cache, **kw)
    assert M.info()["col_cached"] == cache
    y = apply(M, torch.from_numpy(x_np).cuda(), torch.from_numpy(y0_np).cuda(), -1.25, 0.5)
    check(a, x_np, y0_np, -1.25, 0.5, y, dtype, what="col_cache=%d %s %s" % (cache, fmt, kw))
    with pytest.raises(sf.SpmvError):
        M.convert(fmt, col_cache=2)
    M.close()


def test_csr_stage_errors():
    a = MATS["c1"]()
    M = sf.Matrix.from_csr(*to_dev(a), n=a.n)
    for kw in (dict(csr_stage=2), dict(csr_stage=-2), dict(csr_stage=1, subwave=32),
               dict(csr_stage=1, subwave=1), dict(csr_stage=1, csr_rows=2),
               dict(csr_stage=1, csr_kernel="balanced")):
        with pytest.raises(sf.SpmvError):
            M.convert("csr", **kw)
    # auto shape with staging forced stays in the staged range
    M.convert("csr", csr_kernel="vector", csr_stage=1)
    inf = M.info()
    assert inf["csr_stage_slots"] >= 256 and 2 <= inf["subwave"] <= 16 and inf["csr_rows"] == 1
    # the balanced kernel reports no staging
    M.convert("csr", csr_kernel="balanced")
    assert M.info()["csr_stage_slots"] == 0
    M.close()


def test_sell_split_slices():
    """Slices wider than the split width go through column chunks + atomics."""
    n = 9000
    L = np.arange(n) % 13
    L[[5, 700, 701, 4000, 8999]] = [3000, 2900, 257, 8999, 1000]
    a = random_csr(n, seed=45, lens=L)
    x_np, y0_np = vectors(n, 10)
    x = torch.from_numpy(x_np).cuda()
    y0 = torch.from_numpy(y0_np).cuda()
    for sigma in (-1, n, 1024):   # default window (8192 rows), all rows, small windows
        M = sf.Matrix.from_csr(*to_dev(a), n=n).convert("sell64", sort_window=sigma)
        assert M.info()["sort_window"] == {-1: 8192, n: n, 1024: 1024}[sigma]
        for alpha, beta in AB:
            check(a, x_np, y0_np, alpha, beta, apply(M, x, y0, alpha, beta), torch.float64,
                  what="sell split sigma=%d" % sigma)
        M.close()


@pytest.mark.parametrize("name", ["c1", "ragged", "dups_unsorted", "every_len", "nnz0", "n1"])
@pytest.mark.parametrize("dtype", [torch.float64, torch.float32])
def test_layouts_bit_exact(name, dtype):
    a = MATS[name]()
    npdt = np.float64 if dtype == torch.float64 else np.float32
    a = CSR(a.n, a.rowptr, a.col, a.val.astype(npdt))
    M = sf.Matrix.from_csr(*to_dev(a, dtype), n=a.n)
    assert np.array_equal(M.export("rowptr"), a.rowptr.astype(np.int32))
    assert np.array_equal(M.export("col"), a.col)
    assert M.export("val").tobytes() == a.val.tobytes()
    M.convert("ellr")
    oc, ov, ol = oracle.ell(a)
    assert np.array_equal(M.export("ell_col"), oc)
    assert M.export("ell_val").tobytes() == ov.tobytes()
    assert np.array_equal(M.export("ell_len"), ol)
    M.convert("sell64")
    perm, sp, ls, sc, sv = oracle.sell(a)
    assert np.array_equal(M.export("sell_perm"), perm.astype(np.int32))
    assert np.array_equal(M.export("sell_slice_ptr"), sp)
    assert np.array_equal(M.export("sell_len"), ls)
    assert np.array_equal(M.export("sell_col"), sc)
    assert M.export("sell_val").tobytes() == sv.tobytes()
    for sigma, pb in ((0, 0), (1, 0), (64, 0), (128, 0), (1000, 0), (128, 1), (-1, 1)):
        # SELL-64 sorted inside windows of sigma rows (0 keeps the order),
        # in the caller's basis or the permuted one
        M.convert("sell64", sort_window=sigma, permuted_basis=pb)
        assert M.info()["permuted_basis"] == pb
        if sigma < 0:
            sigma = 8192
        perm, sp, ls, sc, sv = oracle.sell(a, sigma=max(sigma, 1), permuted=bool(pb))
        assert M.info()["sort_window"] == (0 if sigma <= 1 or a.n <= 1 else min(sigma, a.n))
        assert np.array_equal(M.export("sell_perm"), perm.astype(np.int32))
        assert np.array_equal(M.export("sell_slice_ptr"), sp)
        assert np.array_equal(M.export("sell_len"), ls)
        assert np.array_equal(M.export("sell_col"), sc)
        assert M.export("sell_val").tobytes() == sv.tobytes()
    for fmt in ("hyb", "hec"):
        for req, sigma in ((-1, 0), (0, 0), (3, 0), (-1, 64), (-1, 1024), (3, 256), (-1, -1)):
            M.convert(fmt, ell_width=req, sort_window=sigma)
            K = M.info()["ell_width"]
            if req >= 0:
                assert K == oracle.hyb_width(a, req)
            else:   # the faster of the two width candidates
                assert K in (oracle.hyb_width(a), max(oracle.hyb_width(a), oracle.regular_width(a)))
            assert M.info()["ell_stride"] == oracle.ELL_BLOCK_SPLIT
            if sigma < 0:   # sorted inside whole blocks when >10% padding would be read
                sigma = oracle.ELL_BLOCK_SPLIT if oracle.ell_pad_fraction(a, K) > 0.1 else 0
            assert M.info()["sort_window"] == (sigma if a.n > 0 else 0)
            oc, ov, ol, op = oracle.ell(a, K, block=oracle.ELL_BLOCK_SPLIT, sigma=sigma,
                                        with_perm=True)
            assert np.array_equal(M.export("ell_col"), oc)
            assert M.export("ell_val").tobytes() == ov.tobytes()
            assert np.array_equal(M.export("ell_len"), ol)
            if sigma > 0 and a.n > 0:
                assert np.array_equal(M.export("ell_perm"), op.astype(np.int32))
            else:
                with pytest.raises(sf.SpmvError):
                    M.export("ell_perm")
            trow, tptr, tcol, tval = oracle.tail(a, K)
            assert M.info()["tail_nnz"] == tcol.size
            if fmt == "hyb":
                assert np.array_equal(M.export("tail_row"), trow)
            else:
                assert np.array_equal(M.export("tail_ptr"), tptr)
            assert np.array_equal(M.export("tail_col"), tcol)
            assert M.export("tail_val").tobytes() == tval.tobytes()


def test_coo_ingest_orders_by_row_then_position():
    a = MATS["dups_unsorted"]()
    rows = np.repeat(np.arange(a.n), a.row_lengths())
    rng = np.random.default_rng(5)
    p = rng.permutation(a.nnz)
    r_t = torch.from_numpy(rows[p].astype(np.int64)).cuda()
    c_t = torch.from_numpy(a.col[p]).cuda()
    v_t = torch.from_numpy(a.val[p]).cuda()
    M = sf.Matrix.from_coo(r_t, c_t, v_t, a.n)
    # expected: stable order by row of the shuffled input
    order = np.argsort(rows[p], kind="stable")
    assert np.array_equal(M.export("rowptr"), a.rowptr.astype(np.int32))
    assert np.array_equal(M.export("col"), a.col[p][order])
    assert M.export("val").tobytes() == a.val[p][order].tobytes()
    x_np, y0_np = vectors(a.n, 11)
    x = torch.from_numpy(x_np).cuda()
    y0 = torch.from_numpy(y0_np).cuda()
    check(a, x_np, y0_np, 1.0, 0.0, apply(M, x, y0, 1.0, 0.0), torch.float64)


def test_invalid_matrices_rejected():
    a = random_csr(200, seed=46, density=0.05)
    rp, col, val = to_dev(a)
    bad = rp.clone()
    bad[0] = 1
    with pytest.raises(sf.SpmvError) as e:
        sf.Matrix.from_csr(bad, col, val)
    assert e.value.code == -2 and "rowptr[0]" in str(e.value)
    bad = rp.clone()
    bad[50] = bad[52] + 1
    with pytest.raises(sf.SpmvError) as e:
        sf.Matrix.from_csr(bad, col, val)
    assert e.value.code == -2
    bad = rp.clone()
    bad[-1] -= 1
    with pytest.raises(sf.SpmvError) as e:
        sf.Matrix.from_csr(bad, col, val)
    assert e.value.code == -2 and "rowptr[n]" in str(e.value)
    badc = col.clone()
    badc[7] = a.n
    with pytest.raises(sf.SpmvError) as e:
        sf.Matrix.from_csr(rp, badc, val)
    assert e.value.code == -2 and "column" in str(e.value)
    badc[7] = -1
    with pytest.raises(sf.SpmvError):
        sf.Matrix.from_csr(rp, badc, val)
    rows = torch.zeros(a.nnz, dtype=torch.int64, device="cuda")
    rows[3] = a.n
    with pytest.raises(sf.SpmvError) as e:
        sf.Matrix.from_coo(rows, col, val, a.n)
    assert e.value.code == -2 and "row" in str(e.value)


def test_footprint_refusal_keeps_handle():
    a = MATS["ragged"]()
    x_np, y0_np = vectors(a.n, 12)
    M = sf.Matrix.from_csr(*to_dev(a), n=a.n).convert("sell64")
    with pytest.raises(sf.SpmvError) as e:
        M.convert("ellr", footprint_budget=1 << 20)
    assert e.value.code == -4
    assert M.info()["format"] == "sell64"
    x = torch.from_numpy(x_np).cuda()
    y0 = torch.from_numpy(y0_np).cuda()
    check(a, x_np, y0_np, 1.0, 0.0, apply(M, x, y0, 1.0, 0.0), torch.float64)
    with pytest.raises(sf.SpmvError) as e:
        M.export("ell_col")
    assert e.value.code == -6


def test_argument_errors_on_device():
    a = MATS["c1"]()
    M = sf.Matrix.from_csr(*to_dev(a), n=a.n)
    buf = torch.zeros(2 * a.n, dtype=torch.float64, device="cuda")
    with pytest.raises(sf.SpmvError) as e:
        M.apply(buf[10:10 + a.n], buf[:a.n])
    assert e.value.code == -1 and "overlap" in str(e.value)
    with pytest.raises(sf.SpmvError) as e:
        M.convert("csr", subwave=3)
    assert e.value.code == -1
    with pytest.raises(TypeError):
        M.apply(torch.zeros(a.n, dtype=torch.float32, device="cuda"),
                torch.zeros(a.n, dtype=torch.float32, device="cuda"))


@pytest.mark.parametrize("fmt", FORMATS)
def test_beta_zero_ignores_nan_y(fmt):
    a = MATS["ragged"]()
    x_np, _ = vectors(a.n, 13)
    M = sf.Matrix.from_csr(*to_dev(a), n=a.n).convert(fmt)
    x = torch.from_numpy(x_np).cuda()
    y = torch.full((a.n,), float("nan"), dtype=torch.float64, device="cuda")
    M.apply(y, x, 1.0, 0.0)
    yn = y.cpu().numpy()
    assert np.all(np.isfinite(yn))
    check(a, x_np, None, 1.0, 0.0, yn, torch.float64)


def test_determinism():
    """Kernels without atomics (vector CSR, ELL-R) repeat bit for bit; the
    others add partial sums with atomics, so only the tolerance holds."""
    a = MATS["long_spans"]()
    x_np, _ = vectors(a.n, 14)
    x = torch.from_numpy(x_np).cuda()
    for fmt, kw in [(f, {}) for f in FORMATS] + [("csr", dict(csr_kernel="vector"))]:
        M = sf.Matrix.from_csr(*to_dev(a), n=a.n).convert(fmt, **kw)
        y1 = torch.zeros(a.n, dtype=torch.float64, device="cuda")
        y2 = torch.zeros_like(y1)
        M.apply(y1, x)
        M.apply(y2, x)
        torch.cuda.synchronize()
        if fmt == "ellr" or (fmt == "csr" and M.info()["csr_kernel"] == "vector"):
            assert torch.equal(y1, y2), fmt
        else:
            ref, sc = oracle.spmv(a, x_np)
            assert oracle.check(y1.cpu().numpy(), ref, sc, 1e-12)[0]
            assert oracle.check(y2.cpu().numpy(), ref, sc, 1e-12)[0]
        M.convert(fmt)  # converting twice gives the same layout
        M.close()


def test_convert_twice_same_arrays():
    """Converting again rebuilds the same layout (the width is pinned: with no
    width given HEC times two candidates, and equal ones may come out either
    way)."""
    a = MATS["ragged"]()
    M = sf.Matrix.from_csr(*to_dev(a), n=a.n)
    for fmt, arrays in [("sell64", ["sell_perm", "sell_col", "sell_val", "sell_slice_ptr"]),
                        ("hec", ["ell_col", "tail_ptr", "tail_col", "tail_val"])]:
        M.convert(fmt)
        kw = dict(ell_width=M.info()["ell_width"]) if fmt == "hec" else {}
        M.convert(fmt, **kw)
        first = [M.export(n).tobytes() for n in arrays]
        M.convert(fmt, **kw)
        assert first == [M.export(n).tobytes() for n in arrays]


def test_convert_releases_its_scratch():
    """Timed conversions borrow a 512 MiB buffer (the cache flush between timed
    launches) and the column-slice candidate's arrays; repeated conversions
    leave the device's free memory where it was."""
    a = MATS["long_spans"]()
    M = sf.Matrix.from_csr(*to_dev(a), n=a.n)
    M.convert("hec")
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for fmt in ["csr", "hec", "hyb", "sell64", "auto", "csr"] * 2:
        M.convert(fmt)
    torch.cuda.synchronize()
    M.convert("hec")
    torch.cuda.synchronize()
    assert abs(torch.cuda.mem_get_info()[0] - free0) < (64 << 20)
    M.close()


def test_stream_copy():
    src = torch.randn(1 << 20, dtype=torch.float64, device="cuda")
    dst = torch.empty_like(src)
    sf.stream_copy(dst, src)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    s2 = torch.arange(1000, dtype=torch.int8, device="cuda")  # 1000 bytes: ragged tail
    d2 = torch.zeros_like(s2)
    sf.stream_copy(d2, s2)
    torch.cuda.synchronize()
    assert torch.equal(d2, s2)
    # the read-only stream (dst NULL) leaves its source as it was
    keep = src.clone()
    sf.stream_read(src)
    sf.stream_read(s2)
    torch.cuda.synchronize()
    assert torch.equal(src, keep) and torch.equal(d2, s2)


def test_apply_on_side_stream():
    a = MATS["ragged"]()
    x_np, _ = vectors(a.n, 15)
    M = sf.Matrix.from_csr(*to_dev(a), n=a.n).convert("hec")
    x = torch.from_numpy(x_np).cuda()
    s = torch.cuda.Stream()
    y = torch.zeros(a.n, dtype=torch.float64, device="cuda")
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        M.apply(y, x)
    s.synchronize()
    check(a, x_np, None, 1.0, 0.0, y.cpu().numpy(), torch.float64)


GRAPH_CASES = [("csr", dict(csr_kernel="vector", csr_stage=1)),
               ("csr", dict(csr_kernel="vector", csr_stage=0)),
               ("csr", dict(csr_kernel="balanced", x_window=0)),
               ("csr", dict(csr_kernel="balanced", x_window=1)),
               ("csr", dict(csr_kernel="xblock")),
               ("ellr", dict(x_window=0)), ("ellr", dict(x_window=1)), ("ellr", dict(ell_groups=4)),
               ("sell64", {}),
               ("hyb", dict(x_window=0)), ("hyb", dict(x_window=1)),
               ("hec", dict(csr_kernel="vector", x_window=0)),
               ("hec", dict(csr_kernel="balanced", x_window=1)),
               ("hyb", dict(csr_kernel="xblock", x_window=0)),
               ("hec", dict(csr_kernel="xblock", x_window=1))]


@pytest.mark.parametrize("fmt,kw", GRAPH_CASES)
def test_apply_in_hip_graph(fmt, kw):
    """apply captured in a HIP graph: every replay, with new x and y written
    by eager work in between, matches the oracle (and the eager apply)."""
    a = _banded() if kw.get("x_window") == 1 else MATS["long_spans"]()
    xs = [vectors(a.n, 60 + r)[0] for r in range(4)]
    _, y0_np = vectors(a.n, 59)
    M = sf.Matrix.from_csr(*to_dev(a), n=a.n).convert(fmt, **kw)
    x = torch.from_numpy(xs[0]).cuda()
    y0 = torch.from_numpy(y0_np).cuda()
    y = y0.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        M.apply(y, x, 1.5, -0.5)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        M.apply(y, x, 1.5, -0.5)
    for r in range(4):
        x.copy_(torch.from_numpy(xs[r]))
        y.copy_(y0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        yg = y.cpu().numpy()
        check(a, xs[r], y0_np, 1.5, -0.5, yg, torch.float64,
              what="graph %s %s replay %d" % (fmt, kw, r))
        ye = apply(M, x, y0, 1.5, -0.5)
        check(a, xs[r], y0_np, 1.5, -0.5, ye, torch.float64, what="eager %s %s" % (fmt, kw))
    del g
    M.close()


@pytest.mark.parametrize("fmt", FORMATS)
def test_concurrent_applies_on_two_streams(fmt):
    """One handle applied on two streams at once (different x and y): apply
    keeps no scratch of its own, so neither result depends on the other."""
    a = MATS["long_spans"]()
    x1, y01 = vectors(a.n, 71)
    x2, y02 = vectors(a.n, 72)
    M = sf.Matrix.from_csr(*to_dev(a), n=a.n).convert(fmt)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    xa, xb = torch.from_numpy(x1).cuda(), torch.from_numpy(x2).cuda()
    ya, yb = torch.from_numpy(y01).cuda(), torch.from_numpy(y02).cuda()
    torch.cuda.synchronize()
    for _ in range(3):   # several rounds, each adding onto y (beta = 1)
        with torch.cuda.stream(s1):
            M.apply(ya, xa, 0.5, 1.0)
        with torch.cuda.stream(s2):
            M.apply(yb, xb, -0.25, 1.0)
    torch.cuda.synchronize()
    # three applies of alpha A x onto y0 equal one apply of 3 alpha
    check(a, x1, y01, 1.5, 1.0, ya.cpu().numpy(), torch.float64, what="stream 1 " + fmt)
    check(a, x2, y02, -0.75, 1.0, yb.cpu().numpy(), torch.float64, what="stream 2 " + fmt)
    M.close()


@pytest.mark.parametrize("fmt,kw", [("csr", {}), ("csr", dict(csr_kernel="xblock")),
                                    ("hyb", {}), ("hyb", dict(csr_kernel="xblock")),
                                    ("hec", {}), ("hec", dict(csr_kernel="xblock"))])
def test_concurrent_applies_scattered_columns(fmt, kw):
    """Applies on two streams at once on a matrix shaped like the power-law
    workload (600,000 rows, lognormal lengths, 64 rows of 20,000-50,000
    entries, uniform columns: x of 4.8 MB read at random), where the default
    CSR and tail choices may take the column-slice kernel: with default options
    and with that kernel forced, every row of both results matches the
    oracle."""
    from gen import c4_powerlaw
    a = c4_powerlaw(n=600_000)
    x1, y01 = vectors(a.n, 73)
    x2, y02 = vectors(a.n, 74)
    M = sf.Matrix.from_csr(*to_dev(a), n=a.n).convert(fmt, **kw)
    key = "csr_kernel" if fmt == "csr" else "tail_kernel"
    if kw:
        assert M.info()[key] == "xblock"
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    xa, xb = torch.from_numpy(x1).cuda(), torch.from_numpy(x2).cuda()
    ya, yb = torch.from_numpy(y01).cuda(), torch.from_numpy(y02).cuda()
    torch.cuda.synchronize()
    for _ in range(4):
        with torch.cuda.stream(s1):
            M.apply(ya, xa, 0.5, 1.0)
        with torch.cuda.stream(s2):
            M.apply(yb, xb, -0.25, 1.0)
    torch.cuda.synchronize()
    what = "%s %s (%s)" % (fmt, kw or "default", M.info()[key])
    check(a, x1, y01, 2.0, 1.0, ya.cpu().numpy(), torch.float64, what="stream 1 " + what)
    check(a, x2, y02, -1.0, 1.0, yb.cpu().numpy(), torch.float64, what="stream 2 " + what)
    M.close()


def _arrow(n=3_000_000, seed=81):
    """Row 0 holds every column; every other row its diagonal and column 0."""
    rng = np.random.default_rng(seed)
    lens = np.full(n, 2, np.int64)
    lens[0] = n
    rowptr = np.concatenate([[0], np.cumsum(lens)])
    col = np.empty(rowptr[-1], np.int32)
    col[:n] = np.arange(n)
    rest = np.arange(1, n, dtype=np.int32)
    col[n::2] = 0
    col[n + 1::2] = rest
    return CSR(n, rowptr, col, rng.standard_normal(rowptr[-1]))


def test_arrow_matrix_every_format():
    """A row as long as the matrix (3 M entries) beside rows of 2: the long row
    goes to the tail, to column chunks or to wide groups, and the conversion
    does not time shapes that would crawl along it.  ELL-R is refused."""
    a = _arrow()
    x_np, y0_np = vectors(a.n, 82)
    x = torch.from_numpy(x_np).cuda()
    y0 = torch.from_numpy(y0_np).cuda()
    M = sf.Matrix.from_csr(*to_dev(a), n=a.n)
    for fmt, kw in (("csr", {}), ("csr", dict(csr_kernel="vector")),
                    ("csr", dict(csr_kernel="vector", csr_stage=1)), ("sell64", {}),
                    ("hyb", {}), ("hec", {}), ("hec", dict(csr_kernel="vector")), ("auto", {})):
        M.convert(fmt, **kw)
        check(a, x_np, y0_np, 0.5, 2.0, apply(M, x, y0, 0.5, 2.0), torch.float64,
              what="arrow %s %s" % (fmt, kw))
    with pytest.raises(sf.SpmvError) as e:
        M.convert("ellr")
    assert e.value.code == -4
    M.close()


def _banded():
    # banded rows (|col - row| up to 12,000: partly beyond the LDS window),
    # a few long rows and 5% far columns; enough rows and entries that the
    # persistent window kernels slide over several tiles / steps
    return gen_c5(n=1_200_000, lo=3, hi=12, frac_long=0.0005, long_len=3000, band=12_000,
                  seed=47)


from gen import c5_fem as gen_c5  # noqa: E402

WINDOW_MATS = dict(MATS, banded=_banded)


@pytest.mark.parametrize("dtype", [torch.float64, torch.float32])
@pytest.mark.parametrize("name", ["c1", "ragged", "every_len", "long_spans", "box27", "nnz0",
                                  "n1", "banded"])
@pytest.mark.parametrize("fmt", ["ellr", "hyb", "hec"])
@pytest.mark.parametrize("win", [1, 0])
def test_x_window_forced(fmt, name, dtype, win):
    a = WINDOW_MATS[name]()
    if dtype == torch.float32:
        a = CSR(a.n, a.rowptr, a.col, a.val.astype(np.float32))
    npdt = np.float64 if dtype == torch.float64 else np.float32
    x_np, y0_np = vectors(a.n, 16)
    x_np, y0_np = x_np.astype(npdt), y0_np.astype(npdt)
    M = sf.Matrix.from_csr(*to_dev(a, dtype), n=a.n)
    kws = [dict()]
    if fmt != "ellr":
        kws.append(dict(ell_width=0))   # whole matrix in the tail
    x = torch.from_numpy(x_np).cuda()
    y0 = torch.from_numpy(y0_np).cuda()
    for kw in kws:
        if fmt == "ellr" and name == "banded":
            kw = dict(footprint_budget=1 << 40)
        M.convert(fmt, x_window=win, **kw)
        assert M.info()["x_window"] == win
        for alpha, beta in AB[:2]:
            y = apply(M, x, y0, alpha, beta)
            rows = None if a.n < 100_000 else np.unique(np.concatenate(
                [np.arange(0, a.n, 97), np.argsort(a.row_lengths())[-200:]]))
            check(a, x_np, y0_np, alpha, beta, y, dtype, rows=rows,
                  what="%s win=%d %s %s" % (fmt, win, kw, name))
    M.close()


def test_x_window_auto_choice():
    """Auto: a candidate when half the entries are within reach, then timed."""
    a = _banded()
    M = sf.Matrix.from_csr(*to_dev(a), n=a.n).convert("hec")
    i = M.info()
    assert 0.7 < i["band_fraction"] < 0.9 and i["x_window"] in (0, 1)
    # far columns everywhere: never a candidate
    far = random_csr(300_000, seed=48, density=2e-5)
    M2 = sf.Matrix.from_csr(*to_dev(far), n=far.n).convert("hyb")
    assert M2.info()["band_fraction"] < 0.5 and M2.info()["x_window"] == 0
    M2.convert("csr", csr_kernel="balanced")
    assert M2.info()["x_window"] == 0
    with pytest.raises(sf.SpmvError):
        M2.convert("hyb", x_window=2)


@pytest.mark.parametrize("dtype", [torch.float64, torch.float32])
@pytest.mark.parametrize("name", list(MATS) + ["banded"])
@pytest.mark.parametrize("win", [0, 1])
def test_csr_balanced(name, dtype, win):
    """The entry-balanced CSR kernel (beta pass, then 512-entry wave chunks
    with a segmented scan and atomics for rows that cross chunks)."""
    a = WINDOW_MATS[name]()
    if dtype == torch.float32:
        a = CSR(a.n, a.rowptr, a.col, a.val.astype(np.float32))
    npdt = np.float64 if dtype == torch.float64 else np.float32
    x_np, y0_np = vectors(a.n, 17)
    x_np, y0_np = x_np.astype(npdt), y0_np.astype(npdt)
    M = sf.Matrix.from_csr(*to_dev(a, dtype), n=a.n).convert("csr", csr_kernel="balanced",
                                                             x_window=win)
    i = M.info()
    assert i["csr_kernel"] == "balanced" and i["format"] == "csr"
    assert i["x_window"] == (win if a.nnz > 0 else 0)
    x = torch.from_numpy(x_np).cuda()
    y0 = torch.from_numpy(y0_np).cuda()
    rows = None if a.n < 100_000 else np.unique(np.concatenate(
        [np.arange(0, a.n, 97), np.argsort(a.row_lengths())[-200:]]))
    for alpha, beta in AB:
        y = apply(M, x, y0, alpha, beta)
        check(a, x_np, y0_np, alpha, beta, y, dtype, rows=rows,
              what="csr balanced win=%d %s a=%g b=%g" % (win, name, alpha, beta))
    if a.n > 0:
        # beta = 0 never reads y: NaNs in y must not survive
        y = torch.full((a.n,), float("nan"), dtype=dtype, device="cuda")
        M.apply(y, x)
        torch.cuda.synchronize()
        check(a, x_np, None, 1.0, 0.0, y.cpu().numpy(), dtype, rows=rows,
              what="csr balanced NaN y %s" % name)
    M.close()


def test_csr_kernel_choice():
    for name in ["c1", "ragged", "long_spans"]:
        a = MATS[name]()
        x_np, y0_np = vectors(a.n, 18)
        M = sf.Matrix.from_csr(*to_dev(a), n=a.n).convert("csr")
        assert M.info()["csr_kernel"] in ("vector", "balanced")
        y = apply(M, torch.from_numpy(x_np).cuda(), torch.from_numpy(y0_np).cuda(), 1.5, -0.5)
        check(a, x_np, y0_np, 1.5, -0.5, y, torch.float64, what="csr auto %s" % name)
        M.convert("csr", csr_kernel="vector")
        assert M.info()["csr_kernel"] == "vector" and M.info()["x_window"] == 0
        # converting to another format and back keeps the handle consistent
        M.convert("hec").convert("csr", csr_kernel="balanced")
        assert M.info()["csr_kernel"] == "balanced"
        y = apply(M, torch.from_numpy(x_np).cuda(), torch.from_numpy(y0_np).cuda(), 1.0, 1.0)
        check(a, x_np, y0_np, 1.0, 1.0, y, torch.float64, what="csr balanced %s" % name)
        with pytest.raises(sf.SpmvError):
            M.convert("csr", csr_kernel=4)
        M.close()


def _scattered():
    # random columns over the whole row range (the x reads the column slices
    # are for), lognormal lengths, a few rows spanning many waves, empty rows
    rng = np.random.default_rng(47)
    n = 50_000
    lens = np.minimum(np.rint(rng.lognormal(np.log(6.0), 1.0, n)).astype(np.int64), n)
    lens[rng.choice(n, 5000, replace=False)] = 0
    lens[rng.choice(n, 4, replace=False)] = [n, 20_000, 4_097, 513]
    return random_csr(n, seed=48, lens=lens)


XBLOCK_MATS = dict(WINDOW_MATS, scattered=_scattered,
                   n7=lambda: random_csr(7, seed=49, lens=np.array([0, 7, 1, 0, 3, 7, 2])))


@pytest.mark.parametrize("dtype", [torch.float64, torch.float32])
@pytest.mark.parametrize("name", list(XBLOCK_MATS))
def test_csr_xblock(name, dtype):
    """CSR by column slices (row ranges summed in LDS slice by slice, each
    range's y written once) against the oracle, and NaNs in y dropped when
    beta = 0."""
    a = XBLOCK_MATS[name]()
    if dtype == torch.float32:
        a = CSR(a.n, a.rowptr, a.col, a.val.astype(np.float32))
    npdt = np.float64 if dtype == torch.float64 else np.float32
    x_np, y0_np = vectors(a.n, 21)
    x_np, y0_np = x_np.astype(npdt), y0_np.astype(npdt)
    M = sf.Matrix.from_csr(*to_dev(a, dtype), n=a.n).convert("csr", csr_kernel="xblock")
    i = M.info()
    assert i["csr_kernel"] == "xblock" and i["format"] == "csr" and i["x_window"] == 0
    assert i["csr_stage_slots"] == 0
    x = torch.from_numpy(x_np).cuda()
    y0 = torch.from_numpy(y0_np).cuda()
    for alpha, beta in AB:
        y = apply(M, x, y0, alpha, beta)
        check(a, x_np, y0_np, alpha, beta, y, dtype,
              what="csr xblock %s a=%g b=%g" % (name, alpha, beta))
    if a.n > 0:
        y = torch.full((a.n,), float("nan"), dtype=dtype, device="cuda")
        M.apply(y, x)
        torch.cuda.synchronize()
        check(a, x_np, None, 1.0, 0.0, y.cpu().numpy(), dtype, what="csr xblock NaN y %s" % name)
        # repeated applies onto the previous result
        for _ in range(2):
            y = apply(M, x, y0, 1.0, 1.0)
            check(a, x_np, y0_np, 1.0, 1.0, y, dtype, what="csr xblock again %s" % name)
    # back to another kernel and format and again: the handle stays consistent
    M.convert("hec").convert("csr", csr_kernel="xblock")
    y = apply(M, x, y0, 0.5, 2.0)
    check(a, x_np, y0_np, 0.5, 2.0, y, dtype, what="csr xblock again %s" % name)
    M.close()


def test_csr_xblock_errors():
    a = MATS["c1"]()
    M = sf.Matrix.from_csr(*to_dev(a), n=a.n)
    for fmt, kw in [("ellr", {}), ("sell64", {}), ("auto", {}), ("hyb", dict(subwave=4)),
                    ("hec", dict(subwave=4)), ("csr", dict(subwave=4)), ("csr", dict(csr_rows=2)),
                    ("csr", dict(csr_stage=1)), ("csr", dict(x_window=1))]:
        with pytest.raises(sf.SpmvError) as e:
            M.convert(fmt, csr_kernel="xblock", **kw)
        assert e.value.code == -1, (fmt, kw)
    M.convert("csr", csr_kernel="xblock")  # the failed calls left it usable
    assert M.info()["csr_kernel"] == "xblock"
    M.close()


@pytest.mark.parametrize("dtype", [torch.float64, torch.float32])
@pytest.mark.parametrize("name", ["c1", "ragged", "every_len", "long_spans", "box27", "nnz0",
                                  "n1", "dups_unsorted", "banded"])
@pytest.mark.parametrize("fmt,sigma,win", [("sell64", 0, -1), ("sell64", 64, -1),
                                           ("sell64", 4096, -1), ("hyb", 64, 0), ("hyb", 1024, 1),
                                           ("hec", 1024, 0), ("hec", 256, 1)])
def test_windowed_sort_parity(fmt, sigma, win, name, dtype):
    """Formats whose rows are sorted only inside windows (y written through
    the permutation; the LDS x window on or off for the sorted ELL part)."""
    a = WINDOW_MATS[name]()
    if dtype == torch.float32:
        a = CSR(a.n, a.rowptr, a.col, a.val.astype(np.float32))
    npdt = np.float64 if dtype == torch.float64 else np.float32
    x_np, y0_np = vectors(a.n, 19)
    x_np, y0_np = x_np.astype(npdt), y0_np.astype(npdt)
    M = sf.Matrix.from_csr(*to_dev(a, dtype), n=a.n).convert(fmt, sort_window=sigma,
                                                             x_window=win)
    x = torch.from_numpy(x_np).cuda()
    y0 = torch.from_numpy(y0_np).cuda()
    rows = None if a.n < 100_000 else np.unique(np.concatenate(
        [np.arange(0, a.n, 97), np.argsort(a.row_lengths())[-200:]]))
    for alpha, beta in AB[:3]:
        y = apply(M, x, y0, alpha, beta)
        check(a, x_np, y0_np, alpha, beta, y, dtype, rows=rows,
              what="%s sort=%d win=%d %s a=%g b=%g" % (fmt, sigma, win, name, alpha, beta))
    M.close()


def test_sort_window_errors():
    a = MATS["ragged"]()
    M = sf.Matrix.from_csr(*to_dev(a), n=a.n)
    for fmt, sigma in (("hyb", 100), ("hec", 2048), ("hyb", 32), ("ellr", 64), ("csr", 64),
                       ("sell64", -2)):
        with pytest.raises(sf.SpmvError):
            M.convert(fmt, sort_window=sigma)
    M.convert("sell64", sort_window=7)   # any window works for SELL-64
    assert M.info()["sort_window"] == 7
    M.close()


@pytest.mark.parametrize("name", ["c1", "ragged", "every_len", "long_spans", "box27", "n1", "nnz0",
                                  "banded"])
def test_auto_format(name):
    """SPMV_AUTO keeps one of the five formats (ELL-R only when its padding is
    at most 1.5x the entries) and applies it exactly like that format."""
    a = WINDOW_MATS[name]()
    x_np, y0_np = vectors(a.n, 20)
    M = sf.Matrix.from_csr(*to_dev(a), n=a.n).convert("hec").convert("auto")
    fmt = M.info()["format"]
    assert fmt in FORMATS
    if oracle.pad64(a.n) * oracle.max_len(a) > 1.5 * max(a.nnz, 1):
        assert fmt != "ellr"
    x = torch.from_numpy(x_np).cuda()
    y0 = torch.from_numpy(y0_np).cuda()
    rows = None if a.n < 100_000 else np.arange(0, a.n, 61)
    for alpha, beta in AB[:2]:
        check(a, x_np, y0_np, alpha, beta, apply(M, x, y0, alpha, beta), torch.float64, rows=rows,
              what="auto -> %s on %s" % (fmt, name))
    # a budget that refuses ELL-R still leaves a choice
    M.convert("auto", footprint_budget=1)
    assert M.info()["format"] != "ellr"
    with pytest.raises(sf.SpmvError):
        M.convert("auto", sort_window=100)
    M.close()


@pytest.mark.parametrize("dtype", [torch.float64, torch.float32])
@pytest.mark.parametrize("name", ["c1", "ragged", "every_len", "long_spans", "dups_unsorted", "n1",
                                  "nnz0", "banded"])
@pytest.mark.parametrize("sigma", [-1, 64, 10 ** 9])
def test_sell_permuted_basis(name, dtype, sigma):
    """apply in the sorted basis: y' = P A P^T x' + beta y' with (P v)[r] =
    v[perm[r]], checked against the oracle in the caller's basis; spmv_permute
    moves vectors there and back exactly."""
    a = WINDOW_MATS[name]()
    if dtype == torch.float32:
        a = CSR(a.n, a.rowptr, a.col, a.val.astype(np.float32))
    npdt = np.float64 if dtype == torch.float64 else np.float32
    x_np, y0_np = vectors(a.n, 21)
    x_np, y0_np = x_np.astype(npdt), y0_np.astype(npdt)
    M = sf.Matrix.from_csr(*to_dev(a, dtype), n=a.n).convert("sell64", sort_window=sigma,
                                                             permuted_basis=1)
    if a.n == 0:
        return
    perm = M.export("sell_perm").astype(np.int64)
    x = torch.from_numpy(x_np).cuda()
    y0 = torch.from_numpy(y0_np).cuda()
    xp = torch.empty_like(x)
    y0p = torch.empty_like(y0)
    M.permute(xp, x)
    M.permute(y0p, y0)
    torch.cuda.synchronize()
    assert np.array_equal(xp.cpu().numpy(), x_np[perm])     # moves values exactly
    back = torch.empty_like(x)
    M.permute(back, xp, inverse=True)
    torch.cuda.synchronize()
    assert np.array_equal(back.cpu().numpy(), x_np)
    rows = None if a.n < 100_000 else np.arange(0, a.n, 53)
    for alpha, beta in AB[:3]:
        yp = apply(M, xp, y0p, alpha, beta)          # sorted basis
        y = np.empty_like(yp)
        y[perm] = yp                                 # back to the caller's basis
        check(a, x_np, y0_np, alpha, beta, y, dtype, rows=rows,
              what="sell permuted sigma=%d %s a=%g b=%g" % (sigma, name, alpha, beta))
    with pytest.raises(sf.SpmvError):
        M.permute(xp, xp)                            # overlap
    M.convert("hyb")
    with pytest.raises(sf.SpmvError):
        M.permute(xp, x)                             # no permutation active
    with pytest.raises(sf.SpmvError):
        M.convert("hyb", permuted_basis=1)
    M.close()


def _short_wide():
    # few rows (under one tile per CU), long rows of mixed length
    rng = np.random.default_rng(49)
    return random_csr(1500, seed=49, lens=rng.integers(200, 3000, 1500))


@pytest.mark.parametrize("dtype", [torch.float64, torch.float32])
@pytest.mark.parametrize("name", ["short_wide", "c1", "ragged", "every_len", "long_spans", "n1",
                                  "nnz0"])
@pytest.mark.parametrize("fmt,kw", [("ellr", {}), ("hyb", dict(ell_width=10 ** 6)),
                                    ("hec", {}), ("hyb", dict(sort_window=1024))])
@pytest.mark.parametrize("groups", [0, 4, 16])
def test_ell_wave_groups(fmt, kw, groups, name, dtype):
    """ELL kernel with several wave groups per 64-row tile (each group every
    G-th column, partial sums joined in LDS)."""
    a = _short_wide() if name == "short_wide" else MATS[name]()
    if dtype == torch.float32:
        a = CSR(a.n, a.rowptr, a.col, a.val.astype(np.float32))
    npdt = np.float64 if dtype == torch.float64 else np.float32
    x_np, y0_np = vectors(a.n, 22)
    x_np, y0_np = x_np.astype(npdt), y0_np.astype(npdt)
    M = sf.Matrix.from_csr(*to_dev(a, dtype), n=a.n).convert(fmt, ell_groups=groups, x_window=0,
                                                             **kw)
    g = M.info()["ell_groups"]
    if groups:
        assert g == groups
    elif name == "short_wide" and fmt == "ellr":
        assert g == 16          # 24 tiles of 64 rows, rows of hundreds of entries
    x = torch.from_numpy(x_np).cuda()
    y0 = torch.from_numpy(y0_np).cuda()
    for alpha, beta in AB[:3]:
        check(a, x_np, y0_np, alpha, beta, apply(M, x, y0, alpha, beta), dtype,
              what="%s %s groups=%d %s" % (fmt, kw, g, name))
    with pytest.raises(sf.SpmvError):
        M.convert(fmt, ell_groups=8)
    M.close()


def _banded_wide():
    # the FEM block's shape at 300,000 rows: rows of 20-40 within +-10,000
    # of the diagonal (5 % uniform), 1 % of rows with 2,000 entries (slices
    # wider than the window kernel's head, cut into chunks), sorted columns
    return gen_c5(n=300_000, seed=51)


SELL_WIN_MATS = dict(WINDOW_MATS, banded_wide=_banded_wide)


@pytest.mark.parametrize("dtype", [torch.float64, torch.float32])
@pytest.mark.parametrize("name", ["c1", "ragged", "every_len", "long_spans", "box27", "nnz0",
                                  "n1", "dups_unsorted", "banded", "banded_wide"])
@pytest.mark.parametrize("sigma,permuted", [(-1, 0), (64, 0), (8192, 0), (0, 0), (-1, 1)])
def test_sell_window(name, dtype, sigma, permuted):
    """SELL-64 with x in the LDS window (forced): narrow slices written with
    alpha s + beta y, the columns of slices wider than 128 past the first 64
    taken as chunks by the tile's waves and added with atomics after a beta
    pass over their rows.  Any sort window works (the window's reach only
    decides how many x reads go to global memory); -1 takes 1,024 rows."""
    a = SELL_WIN_MATS[name]()
    if dtype == torch.float32:
        a = CSR(a.n, a.rowptr, a.col, a.val.astype(np.float32))
    npdt = np.float64 if dtype == torch.float64 else np.float32
    x_np, y0_np = vectors(a.n, 23)
    x_np, y0_np = x_np.astype(npdt), y0_np.astype(npdt)
    M = sf.Matrix.from_csr(*to_dev(a, dtype), n=a.n).convert(
        "sell64", x_window=1, sort_window=sigma, permuted_basis=permuted)
    i = M.info()
    assert i["x_window"] == (1 if a.n > 0 else 0)
    if sigma == -1 and a.n > 1024:
        assert i["sort_window"] == 1024
    x = torch.from_numpy(x_np).cuda()
    y0 = torch.from_numpy(y0_np).cuda()
    perm = M.export("sell_perm").astype(np.int64) if a.n else np.zeros(0, np.int64)
    for alpha, beta in AB:
        if permuted:
            xp, y0p = torch.empty_like(x), torch.empty_like(y0)
            M.permute(xp, x)
            M.permute(y0p, y0)
            yp = apply(M, xp, y0p, alpha, beta)
            y = np.empty_like(yp)
            y[perm] = yp
        else:
            y = apply(M, x, y0, alpha, beta)
        check(a, x_np, y0_np, alpha, beta, y, dtype,
              what="sell window sigma=%d perm=%d %s a=%g b=%g" % (sigma, permuted, name, alpha,
                                                                  beta))
    if a.n > 0 and not permuted:
        y = torch.full((a.n,), float("nan"), dtype=dtype, device="cuda")
        M.apply(y, x)
        torch.cuda.synchronize()
        check(a, x_np, None, 1.0, 0.0, y.cpu().numpy(), dtype, what="sell window NaN y " + name)
    M.close()


def test_sell_window_layout_and_choice():
    """The window's SELL layout is the oracle's SELL-64 with 1,024-row sort
    windows, byte for byte; the automatic choice takes the window for the
    banded FEM-like matrix only when it is faster, and never for far columns."""
    a = _banded_wide()
    M = sf.Matrix.from_csr(*to_dev(a), n=a.n).convert("sell64", x_window=1)
    perm, sp, ls, sc, sv = oracle.sell(a, sigma=1024)
    assert np.array_equal(M.export("sell_perm"), perm.astype(np.int32))
    assert np.array_equal(M.export("sell_slice_ptr"), sp)
    assert np.array_equal(M.export("sell_len"), ls)
    assert np.array_equal(M.export("sell_col"), sc)
    assert M.export("sell_val").tobytes() == sv.tobytes()
    M.convert("sell64")       # auto: either layout, always correct
    i = M.info()
    assert i["x_window"] in (0, 1) and i["band_fraction"] > 0.8
    assert i["sort_window"] == (1024 if i["x_window"] else 8192)
    x_np, y0_np = vectors(a.n, 24)
    y = apply(M, torch.from_numpy(x_np).cuda(), torch.from_numpy(y0_np).cuda(), 1.5, -0.5)
    check(a, x_np, y0_np, 1.5, -0.5, y, torch.float64, what="sell auto window")
    far = random_csr(300_000, seed=48, density=2e-5)
    M2 = sf.Matrix.from_csr(*to_dev(far), n=far.n).convert("sell64")
    assert M2.info()["x_window"] == 0 and M2.info()["sort_window"] == 8192
    M.close()
    M2.close()
