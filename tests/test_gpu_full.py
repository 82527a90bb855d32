"""GPU parity at the five workloads' full sizes, in the launch configuration the
benchmark times: every format is built from the full matrix and applied to the
full vector; the oracle checks a sample of rows (random rows, the longest
rows, both ends).  ELL-R of the power-law matrix (~2.4 TB padded) must be
refused with FOOTPRINT."""
import sys
import time

import numpy as np
import pytest
import torch

import gen

from gpu_util import FORMATS, apply, check, sample_rows, to_dev

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


def log(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.mark.parametrize("name,dtype", CASES, ids=["%s-%s" % (n, str(d)[6:]) for n, d in CASES])
def test_full_size(name, dtype):
    t0 = time.time()
    npdt = np.float64 if dtype == torch.float64 else np.float32
    a, x_np, y0_np, _ = gen.by_name(name, npdt)
    log("[full] %s %s: n=%d nnz=%d generated in %.1fs" % (name, dtype, a.n, a.nnz,
                                                           time.time() - t0))
    rows = None if a.n <= 100_000 else sample_rows(a)
    M = sf.Matrix.from_csr(*to_dev(a, dtype), n=a.n)
    torch.cuda.empty_cache()
    x = torch.from_numpy(x_np).cuda()
    y0 = torch.from_numpy(y0_np).cuda()
    for fmt in FORMATS:
        try:
            M.convert(fmt)
        except sf.SpmvError as e:
            assert name.startswith("c4") and fmt == "ellr" and e.code == -4, str(e)
            log("[full]   %s refused: %s" % (fmt, e))
            continue
        assert not (name.startswith("c4") and fmt == "ellr"), "ELL-R of C4 must be refused"
        for alpha, beta in [(1.0, 0.0), (-1.5, 0.5)]:
            y = apply(M, x, y0, alpha, beta)
            w = check(a, x_np, y0_np, alpha, beta, y, dtype, rows=rows,
                      what="%s %s a=%g b=%g" % (name, fmt, alpha, beta))
        log("[full]   %s ok (worst err/tol %.3g) %s" % (fmt, w, M.info()))
    M.close()
    torch.cuda.empty_cache()
