"""Helpers for the GPU tests: upload a generated matrix, run one format, and
compare with the CPU oracle at the per-entry tolerance

    |y_gpu_i - y_ref_i| <= tol * (|alpha| sum_j |a_ij x_j| + |beta y_i|),

tol = 1e-12 for fp64 and 1e-5 for fp32 (entries whose scale is 0 must match
exactly)."""
import numpy as np
import torch

import oracle

FORMATS = ["csr", "ellr", "sell64", "hyb", "hec"]
TOL = {torch.float64: 1e-12, torch.float32: 1e-5}
AB = [(1.0, 0.0), (1.5, -0.5), (0.0, 2.0), (-1.0, 1.0)]


def to_dev(a, dtype=torch.float64):
    npdt = np.float64 if dtype == torch.float64 else np.float32
    rp = torch.from_numpy(np.ascontiguousarray(a.rowptr, np.int64)).cuda()
    col = torch.from_numpy(np.ascontiguousarray(a.col, np.int32)).cuda()
    val = torch.from_numpy(np.ascontiguousarray(a.val, npdt)).cuda()
    return rp, col, val


def apply(M, x, y0, alpha, beta):
    """y = alpha A x + beta y0 on the GPU (y0 copied first); returns numpy."""
    y = y0.clone()
    M.apply(y, x, alpha, beta)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def check(a, x_np, y0_np, alpha, beta, y_gpu, dtype, rows=None, what=""):
    """Assert the oracle tolerance on all rows (or the listed rows)."""
    ref, scale = oracle.spmv(a, x_np, y0_np, alpha, beta, rows=rows, nthreads=0)
    yg = y_gpu if rows is None else y_gpu[rows]
    ok, worst, k = oracle.check(yg, ref, scale, TOL[dtype])
    assert ok, "%s: worst |err|/(tol*scale) = %.3g at %s (gpu %r ref %r scale %r)" % (
        what, worst, k if rows is None else rows[k], float(yg[k]), float(ref[k]), float(scale[k]))
    return worst
