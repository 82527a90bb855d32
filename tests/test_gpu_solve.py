"""Krylov solvers over the GPU product (conjugate gradients, BiCGSTAB)
against the oracle's textbook solvers and dense solves: the consumer of SpMV
("Development of Krylov and AMG linear solvers...", Sect. 3)."""
import math

import numpy as np
import pytest
import torch

import oracle
from gen import c1_laplace2d, stencil, vectors

from gpu_util import FORMATS, to_dev

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import sparse_formats_amd as sf


def _system(a, seed):
    x_true = np.random.default_rng(seed).standard_normal(a.n)
    b = oracle.spmv(a, x_true)[0]
    return x_true, b


@pytest.mark.parametrize("fmt,kw", [(f, {}) for f in FORMATS] + [("csr", dict(csr_kernel="xblock"))])
def test_cg_laplacian(fmt, kw):
    a = c1_laplace2d()
    x_true, b = _system(a, 1)
    xo, it_o, rel_o = oracle.cg(a, b, rtol=1e-10, max_iter=2000)
    M = sf.Matrix.from_csr(*to_dev(a), n=a.n).convert(fmt, **kw)
    x, info = M.solve(torch.from_numpy(b).cuda(), rtol=1e-10, max_iter=2000)
    xg = x.cpu().numpy()
    assert info["converged"] and info["rel_residual"] <= 1e-10
    assert abs(info["iterations"] - it_o) <= 3, (info, it_o)
    assert np.linalg.norm(xg - x_true) <= 1e-6 * np.linalg.norm(x_true)
    assert np.linalg.norm(xg - xo) <= 1e-6 * np.linalg.norm(xo)
    # the true residual agrees with the recurred one
    res = oracle.spmv(a, xg, b, -1.0, 1.0)[0]
    assert np.linalg.norm(res) <= 1e-9 * np.linalg.norm(b)
    M.close()


def test_cg_exact_cases():
    a = c1_laplace2d()
    M = sf.Matrix.from_csr(*to_dev(a), n=a.n).convert("ellr")
    r, c = np.divmod(np.arange(a.n), 64)
    v = np.sin(2 * math.pi * (r + 1) / 65) * np.sin(3 * math.pi * (c + 1) / 65)
    lam = 4 - 2 * math.cos(2 * math.pi / 65) - 2 * math.cos(3 * math.pi / 65)
    x, info = M.solve(torch.from_numpy(v).cuda(), rtol=1e-12)
    assert info["iterations"] == 1
    assert np.allclose(x.cpu().numpy(), v / lam, rtol=0, atol=1e-12)
    # zero right-hand side: no iteration, x stays 0
    x0, info0 = M.solve(torch.zeros(a.n, dtype=torch.float64, device="cuda"))
    assert info0["iterations"] == 0 and info0["converged"] and not x0.any()
    # the cap is honoured and reported
    b = torch.from_numpy(_system(a, 2)[1]).cuda()
    _, info5 = M.solve(b, rtol=1e-10, max_iter=5)
    assert info5["iterations"] == 5 and not info5["converged"]
    # deterministic: ELL-R adds no atomics and the inner products reduce in a fixed order
    x1, _ = M.solve(b, rtol=1e-10, max_iter=300)
    x2, _ = M.solve(b, rtol=1e-10, max_iter=300)
    assert torch.equal(x1, x2)
    with pytest.raises(sf.SpmvError):
        M.solve(b, method="cg", max_iter=0)
    with pytest.raises(sf.SpmvError):
        M.solve(b, x=b)           # x and b overlap
    M.close()


@pytest.mark.parametrize("fmt,kw", [("csr", {}), ("sell64", {}), ("hec", {}),
                                    ("csr", dict(csr_kernel="xblock"))])
def test_bicgstab_nonsymmetric_stencil(fmt, kw):
    # 27-point stencil with independent noise per entry: not symmetric
    a = stencil((13, 11, 9), "box", 26.0, -1.0, noise=1e-2, seed=3)
    x_true, b = _system(a, 4)
    D = np.zeros((a.n, a.n))
    for i in range(a.n):
        s, e = a.rowptr[i], a.rowptr[i + 1]
        np.add.at(D[i], a.col[s:e], a.val[s:e])
    assert not np.allclose(D, D.T)
    xo, it_o, rel_o = oracle.bicgstab(a, b, rtol=1e-11)
    M = sf.Matrix.from_csr(*to_dev(a), n=a.n).convert(fmt, **kw)
    x, info = M.solve(torch.from_numpy(b).cuda(), method="bicgstab", rtol=1e-11)
    xg = x.cpu().numpy()
    assert info["converged"] and abs(info["iterations"] - it_o) <= 3, (info, it_o)
    assert np.allclose(xg, np.linalg.solve(D, b), rtol=0, atol=1e-8 * np.abs(x_true).max())
    M.close()


def test_cg_fp32():
    a = c1_laplace2d()
    x_true, b = _system(a, 5)
    M = sf.Matrix.from_csr(*to_dev(a, torch.float32), n=a.n).convert("hyb")
    x, info = M.solve(torch.from_numpy(b.astype(np.float32)).cuda(), rtol=1e-5, max_iter=3000)
    assert info["converged"] and x.dtype == torch.float32
    xg = x.cpu().numpy().astype(np.float64)
    assert np.linalg.norm(xg - x_true) <= 5e-2 * np.linalg.norm(x_true)
    M.close()
