"""Python binding of the MI355X sparse matrix-vector library.

Argument marshalling only: every step of create / convert / apply runs in the
HIP library ``libspmv_amd.so`` (C ABI in ``include/spmv_amd.h``).  PyTorch
supplies device memory (tensors) and streams; the library is loaded after
torch so that both use torch's HIP runtime.  If the library has not been
built, importing this package raises ImportError -- there is no fallback.

    import torch, sparse_formats_amd as sf
    A = sf.Matrix.from_csr(rowptr, col, val)     # device tensors
    A.convert("sell64")
    A.apply(y, x, alpha=1.0, beta=0.0)           # on the current torch stream
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

__all__ = ["Matrix", "SpmvError", "FORMATS", "CSR_KERNELS", "ARRAYS", "stream_copy", "stream_read",
           "lib_path", "version"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libspmv_amd.so")

FORMATS = {"csr": 0, "ellr": 1, "sell64": 2, "hyb": 3, "hec": 4, "auto": 5}
CSR_KERNELS = {"auto": 0, "vector": 1, "balanced": 2, "xblock": 3}
ARRAYS = {
    "rowptr": (0, np.int32), "col": (1, np.int32), "val": (2, None),
    "ell_col": (3, np.int32), "ell_val": (4, None), "ell_len": (5, np.int32),
    "sell_perm": (6, np.int32), "sell_slice_ptr": (7, np.int64), "sell_len": (8, np.int32),
    "sell_col": (9, np.int32), "sell_val": (10, None),
    "tail_row": (11, np.int32), "tail_ptr": (12, np.int32), "tail_col": (13, np.int32),
    "tail_val": (14, None), "ell_perm": (15, np.int32),
}
_DTYPE = {torch.float32: 1, torch.float64: 2}
_NP = {1: np.float32, 2: np.float64}
_ERRORS = {-1: "INVALID_ARG", -2: "INVALID_MATRIX", -3: "NO_MEMORY", -4: "FOOTPRINT",
           -5: "HIP", -6: "STATE"}


class SpmvError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("%s (%d): %s" % (_ERRORS.get(code, "?"), code, msg))
        self.code = code
        self.name = _ERRORS.get(code, "?")


class _ConvertOpts(ctypes.Structure):
    _fields_ = [("ell_width", ctypes.c_int32), ("subwave", ctypes.c_int32),
                ("x_window", ctypes.c_int32), ("csr_rows", ctypes.c_int32),
                ("csr_kernel", ctypes.c_int32), ("sort_window", ctypes.c_int32),
                ("permuted_basis", ctypes.c_int32), ("ell_groups", ctypes.c_int32),
                ("footprint_budget_bytes", ctypes.c_uint64), ("csr_stage", ctypes.c_int32),
                ("col_cache", ctypes.c_int32)]


class _SolveOpts(ctypes.Structure):
    _fields_ = [("method", ctypes.c_int32), ("max_iter", ctypes.c_int32), ("rtol", ctypes.c_double)]


class _SolveInfo(ctypes.Structure):
    _fields_ = [("iterations", ctypes.c_int32), ("converged", ctypes.c_int32),
                ("rel_residual", ctypes.c_double)]


class _Info(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("nnz", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("format", ctypes.c_int32), ("max_len", ctypes.c_int32),
                ("ell_width", ctypes.c_int32), ("tail_nnz", ctypes.c_int64),
                ("ell_stride", ctypes.c_int64), ("slots", ctypes.c_int64),
                ("subwave", ctypes.c_int32), ("nslices", ctypes.c_int32),
                ("footprint_bytes", ctypes.c_uint64), ("x_window", ctypes.c_int32),
                ("csr_rows", ctypes.c_int32), ("csr_kernel", ctypes.c_int32),
                ("permuted_basis", ctypes.c_int32), ("ell_groups", ctypes.c_int32),
                ("sort_window", ctypes.c_int32),
                ("band_fraction", ctypes.c_double),
                ("ell_rows", ctypes.c_int64), ("csr_stage_slots", ctypes.c_int32),
                ("tail_kernel", ctypes.c_int32), ("tail_subwave", ctypes.c_int32),
                ("tail_rows", ctypes.c_int32), ("tail_stage_slots", ctypes.c_int32),
                ("col_cached", ctypes.c_int32), ("ell_head", ctypes.c_int32),
                ("ell_long_rows", ctypes.c_int64)]


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError("libspmv_amd.so is not built (run sparse_formats_amd.build.build())")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.spmv_create.argtypes = [ctypes.POINTER(P), I, I64, I64, P, P, P, I, P]
    lib.spmv_convert.argtypes = [P, I, ctypes.POINTER(_ConvertOpts)]
    lib.spmv_apply.argtypes = [P, P, P, D, D, P]
    lib.spmv_permute.argtypes = [P, P, P, I, P]
    lib.spmv_solve.argtypes = [P, P, P, ctypes.POINTER(_SolveOpts), ctypes.POINTER(_SolveInfo), P]
    lib.spmv_solve_noalloc.argtypes = [P, P, P, ctypes.POINTER(_SolveOpts),
                                       ctypes.POINTER(_SolveInfo), P]
    lib.spmv_destroy.argtypes = [P]
    lib.spmv_info.argtypes = [P, ctypes.POINTER(_Info)]
    lib.spmv_export.argtypes = [P, I, P, I64, ctypes.POINTER(I64)]
    lib.spmv_stream_copy.argtypes = [P, P, I64, P]
    lib.spmv_last_error.restype = ctypes.c_char_p
    lib.spmv_version.restype = ctypes.c_char_p
    for f in ("spmv_create", "spmv_convert", "spmv_apply", "spmv_destroy", "spmv_info",
              "spmv_export", "spmv_stream_copy", "spmv_permute", "spmv_solve",
              "spmv_solve_noalloc"):
        getattr(lib, f).restype = I
    return lib


_lib = _load()


def lib_path() -> str:
    return _LIB_PATH


def version() -> str:
    return _lib.spmv_version().decode()


def _check(code: int):
    if code != 0:
        raise SpmvError(code, _lib.spmv_last_error().decode())


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dev(t, dtype, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a CUDA (HIP) tensor" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr() if t.numel() else None


class Matrix:
    """A sparse matrix resident on the current GPU, owned by the HIP library."""

    def __init__(self, handle, n, nnz, dtype):
        self._h = handle
        self.n = n
        self.nnz = nnz
        self.dtype = dtype

    @classmethod
    def from_csr(cls, rowptr, col, val, n: int | None = None, stream=None) -> "Matrix":
        """rowptr int64[n+1], col int32[nnz], val float32/float64[nnz] on the GPU."""
        n = rowptr.numel() - 1 if n is None else int(n)
        if rowptr.numel() != n + 1:
            raise ValueError("rowptr must have n + 1 entries")
        nnz = col.numel()
        if val.numel() != nnz:
            raise ValueError("col and val differ in length")
        dt = _DTYPE.get(val.dtype)
        if dt is None:
            raise TypeError("val must be float32 or float64")
        h = ctypes.c_void_p()
        _check(_lib.spmv_create(ctypes.byref(h), 0, n, nnz, _dev(rowptr, torch.int64, "rowptr"),
                                _dev(col, torch.int32, "col"), _dev(val, None, "val"), dt,
                                _stream(stream)))
        return cls(h, n, nnz, val.dtype)

    @classmethod
    def from_coo(cls, row, col, val, n: int, stream=None) -> "Matrix":
        """row int64[nnz], col int32[nnz], val[nnz] on the GPU, any entry order."""
        nnz = col.numel()
        if row.numel() != nnz or val.numel() != nnz:
            raise ValueError("row, col and val differ in length")
        dt = _DTYPE.get(val.dtype)
        if dt is None:
            raise TypeError("val must be float32 or float64")
        h = ctypes.c_void_p()
        _check(_lib.spmv_create(ctypes.byref(h), 1, int(n), nnz, _dev(row, torch.int64, "row"),
                                _dev(col, torch.int32, "col"), _dev(val, None, "val"), dt,
                                _stream(stream)))
        return cls(h, int(n), nnz, val.dtype)

    def convert(self, fmt: str, ell_width: int = -1, subwave: int = 0, x_window: int = -1,
                footprint_budget: int = 0, csr_rows: int = 0,
                csr_kernel: str = "auto", sort_window: int = -1,
                permuted_basis: int = 0, ell_groups: int = 0, csr_stage: int = -1,
                col_cache: int = -1) -> "Matrix":
        """Build `fmt` on the device and make it active (options as in spmv_convert_opts;
        csr_kernel is "auto", "vector", "balanced" or "xblock")."""
        if fmt not in FORMATS:
            raise ValueError("unknown format %r (one of %s)" % (fmt, ", ".join(FORMATS)))
        ck = CSR_KERNELS.get(csr_kernel, csr_kernel)
        o = _ConvertOpts(int(ell_width), int(subwave), int(x_window), int(csr_rows), int(ck),
                         int(sort_window), int(permuted_basis), int(ell_groups),
                         int(footprint_budget), int(csr_stage), int(col_cache))
        _check(_lib.spmv_convert(self._h, FORMATS[fmt], ctypes.byref(o)))
        return self

    def apply(self, y, x, alpha: float = 1.0, beta: float = 0.0, stream=None):
        """y = alpha * A x + beta * y on the given (default: current) torch stream."""
        for t, nm in ((y, "y"), (x, "x")):
            if t.numel() != self.n:
                raise ValueError("%s must have n = %d entries" % (nm, self.n))
        _check(_lib.spmv_apply(self._h, _dev(y, self.dtype, "y"), _dev(x, self.dtype, "x"),
                               float(alpha), float(beta), _stream(stream)))
        return y

    def permute(self, dst, src, inverse: bool = False, stream=None):
        """Move a vector between the caller's basis and the sorted basis of the
        active SELL-64 format: dst[r] = src[perm[r]], or dst[perm[r]] = src[r]
        when inverse."""
        for t, nm in ((dst, "dst"), (src, "src")):
            if t.numel() != self.n:
                raise ValueError("%s must have n = %d entries" % (nm, self.n))
        _check(_lib.spmv_permute(self._h, _dev(dst, self.dtype, "dst"),
                                 _dev(src, self.dtype, "src"), 1 if inverse else 0,
                                 _stream(stream)))
        return dst

    def solve(self, b, x=None, method: str = "cg", rtol: float = 1e-10, max_iter: int = 1000,
              stream=None, noalloc: bool = False):
        """Solve A x = b with the active format (method "cg" for symmetric
        positive definite A, "bicgstab" otherwise).  x: initial guess, updated
        in place (zeros when None).  noalloc: run spmv_solve_noalloc (the
        library's fixed per-GPU workspace, no device allocation).  Returns
        (x, info dict)."""
        import torch
        if b.numel() != self.n:
            raise ValueError("b must have n = %d entries" % self.n)
        if x is None:
            x = torch.zeros_like(b)
        o = _SolveOpts({"cg": 0, "bicgstab": 1}[method], int(max_iter), float(rtol))
        info = _SolveInfo()
        fn = _lib.spmv_solve_noalloc if noalloc else _lib.spmv_solve
        _check(fn(self._h, _dev(x, self.dtype, "x"), _dev(b, self.dtype, "b"),
                  ctypes.byref(o), ctypes.byref(info), _stream(stream)))
        return x, {"iterations": info.iterations, "converged": bool(info.converged),
                   "rel_residual": info.rel_residual}

    def info(self) -> dict:
        i = _Info()
        _check(_lib.spmv_info(self._h, ctypes.byref(i)))
        d = {k: getattr(i, k) for k, _ in _Info._fields_}
        d["format"] = [k for k, v in FORMATS.items() if v == d["format"]][0]
        d["csr_kernel"] = [k for k, v in CSR_KERNELS.items() if v == d["csr_kernel"]][0]
        d["tail_kernel"] = [k for k, v in CSR_KERNELS.items() if v == d["tail_kernel"]][0]
        return d

    def export(self, name: str) -> np.ndarray:
        """Copy one of the library's arrays to a numpy array (synchronous)."""
        aid, npt = ARRAYS[name]
        npt = npt or _NP[_DTYPE[self.dtype]]
        nb = ctypes.c_int64()
        _check(_lib.spmv_export(self._h, aid, None, 0, ctypes.byref(nb)))
        out = np.empty(nb.value // np.dtype(npt).itemsize, dtype=npt)
        _check(_lib.spmv_export(self._h, aid, out.ctypes.data_as(ctypes.c_void_p),
                                out.nbytes, ctypes.byref(nb)))
        return out

    def close(self):
        h = getattr(self, "_h", None)
        if h:
            self._h = None   # released even when destroy reports an earlier device error
            _check(_lib.spmv_destroy(h))

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def stream_read(src, stream=None):
    """Read src with the library's read-only streaming kernel (nothing written)."""
    _check(_lib.spmv_stream_copy(None, _dev(src, None, "src"), src.numel() * src.element_size(),
                                 _stream(stream)))


def stream_copy(dst, src, stream=None):
    """dst <- src with the library's streaming copy kernel (same byte count)."""
    nb = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nb:
        raise ValueError("dst smaller than src")
    _check(_lib.spmv_stream_copy(_dev(dst, None, "dst"), _dev(src, None, "src"), nb,
                                 _stream(stream)))
