"""The C-ABI library loads on a machine without a GPU, exports every entry
point its header declares, and rejects bad arguments before touching the
device (no compute call is made here)."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spmv_amd.h")
# SPMV_ABI_LIB: a build of the same sources with the host code under the
# sanitizers (tests/test_host_sanitizers.py runs this file against it)
LIB = os.environ.get("SPMV_ABI_LIB") or os.path.join(ROOT, "sparse_formats_amd", "libspmv_amd.so")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(spmv_\w+)\s*\(", src, re.M)))


def enum_values():
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return {k: int(v) for k, v in re.findall(r"\b(SPMV_\w+)\s*=\s*(-?\d+)", src)}


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libspmv_amd.so is not built")
    lib = ctypes.CDLL(LIB)
    lib.spmv_last_error.restype = ctypes.c_char_p
    return lib


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 9, names
    for n in ["spmv_create", "spmv_convert", "spmv_apply", "spmv_destroy", "spmv_info",
              "spmv_export", "spmv_stream_copy", "spmv_last_error", "spmv_version"]:
        assert n in names
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (spmv_\w+)", out))
    assert set(names) <= exported


def test_header_compiles_as_c(tmp_path):
    c = tmp_path / "t.c"
    c.write_text('#include "spmv_amd.h"\nint main(void){spmv_convert_opts o={-1,0,-1,0,0};'
                 'spmv_info_t i; (void)o; (void)i; return SPMV_OK;}\n')
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER),
                        "-c", str(c), "-o", str(tmp_path / "t.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_struct_layouts_match_binding(tmp_path):
    """Sizes and field offsets of the option and info structs as gcc lays them
    out agree with the Python binding's ctypes mirrors."""
    sys.path.insert(0, ROOT)
    import sparse_formats_amd as sf
    mirrors = {"spmv_convert_opts": sf._ConvertOpts, "spmv_info_t": sf._Info,
               "spmv_solve_opts": sf._SolveOpts, "spmv_solve_info": sf._SolveInfo}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "spmv_amd.h"',
             'int main(void){']
    for cname, py in mirrors.items():
        lines.append('printf("%s size %%zu\\n", sizeof(%s));' % (cname, cname))
        for f, _ in py._fields_:
            lines.append('printf("%s %s %%zu\\n", offsetof(%s, %s));' % (cname, f, cname, f))
    lines.append('return 0;}')
    c = tmp_path / "layout.c"
    c.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    r = subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(c), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    got = {}
    for line in subprocess.run([str(exe)], capture_output=True, text=True).stdout.splitlines():
        a, b, v = line.split()
        got[(a, b)] = int(v)
    for cname, py in mirrors.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)


def test_enum_values_match_binding():
    sys.path.insert(0, ROOT)
    ev = enum_values()
    assert ev["SPMV_OK"] == 0 and ev["SPMV_ERR_INVALID_ARG"] == -1
    assert ev["SPMV_ERR_FOOTPRINT"] == -4 and ev["SPMV_ERR_STATE"] == -6
    fm = {"csr": ev["SPMV_CSR"], "ellr": ev["SPMV_ELLR"], "sell64": ev["SPMV_SELL64"],
          "hyb": ev["SPMV_HYB"], "hec": ev["SPMV_HEC"]}
    assert fm == {"csr": 0, "ellr": 1, "sell64": 2, "hyb": 3, "hec": 4}
    assert ev["SPMV_AUTO"] == 5 and ev["SPMV_CSR_BALANCED"] == 2 and ev["SPMV_A_ELL_PERM"] == 15
    assert ev["SPMV_A_TAIL_VAL"] == 14 and ev["SPMV_A_SELL_SLICE_PTR"] == 7
    import sparse_formats_amd as sf
    assert sf.CSR_KERNELS == {"auto": ev["SPMV_CSR_AUTO"], "vector": ev["SPMV_CSR_VECTOR"],
                              "balanced": ev["SPMV_CSR_BALANCED"], "xblock": ev["SPMV_CSR_XBLOCK"]}


def _create(lib, out, kind=0, n=4, nnz=4, rowidx=None, col=None, val=None, dtype=2):
    P = ctypes.c_void_p
    lib.spmv_create.argtypes = [P, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, P, P, P,
                                ctypes.c_int, P]
    return lib.spmv_create(out, kind, n, nnz, rowidx, col, val, dtype, None)


def test_create_argument_errors(lib):
    h = ctypes.c_void_p()
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: the checks fail first
    assert _create(lib, None) == -1 and b"out" in lib.spmv_last_error()
    assert _create(lib, ctypes.byref(h), kind=7) == -1
    assert _create(lib, ctypes.byref(h), dtype=3) == -1
    assert _create(lib, ctypes.byref(h), n=-1) == -1
    assert _create(lib, ctypes.byref(h), nnz=-5) == -1
    assert _create(lib, ctypes.byref(h), nnz=2 ** 31, rowidx=fake, col=fake, val=fake) == -1
    assert _create(lib, ctypes.byref(h), nnz=2 ** 31 - 65536, rowidx=fake, col=fake,
                   val=fake) == -1                      # past the headroom of the entry indices
    assert _create(lib, ctypes.byref(h), n=2 ** 31 - 1, rowidx=fake) == -1
    assert _create(lib, ctypes.byref(h), n=2 ** 31, rowidx=fake) == -1
    assert _create(lib, ctypes.byref(h), rowidx=None, col=fake, val=fake) == -1
    assert _create(lib, ctypes.byref(h), rowidx=fake, col=None, val=fake) == -1
    assert _create(lib, ctypes.byref(h), kind=1, rowidx=fake, col=fake, val=None) == -1
    assert h.value is None


def test_null_handle_errors(lib):
    P = ctypes.c_void_p
    lib.spmv_convert.argtypes = [P, ctypes.c_int, P]
    lib.spmv_apply.argtypes = [P, P, P, ctypes.c_double, ctypes.c_double, P]
    lib.spmv_info.argtypes = [P, P]
    lib.spmv_export.argtypes = [P, ctypes.c_int, P, ctypes.c_int64, P]
    lib.spmv_destroy.argtypes = [P]
    lib.spmv_stream_copy.argtypes = [P, P, ctypes.c_int64, P]
    assert lib.spmv_convert(None, 0, None) == -6
    assert lib.spmv_apply(None, None, None, 1.0, 0.0, None) == -6
    assert lib.spmv_info(None, None) == -6
    assert lib.spmv_export(None, 0, None, 0, None) == -6
    lib.spmv_permute.argtypes = [P, P, P, ctypes.c_int, P]
    assert lib.spmv_permute(None, None, None, 0, None) == -6
    assert lib.spmv_destroy(None) == 0
    # copy: misaligned, negative, overlapping
    assert lib.spmv_stream_copy(P(0x1008), P(0x2000), 16, None) == -1
    assert lib.spmv_stream_copy(P(0x1000), P(0x2000), -1, None) == -1
    assert lib.spmv_stream_copy(P(0x1000), P(0x1010), 64, None) == -1
    assert b"overlap" in lib.spmv_last_error()
    # read-only stream (dst NULL): src still required and aligned
    assert lib.spmv_stream_copy(None, None, 16, None) == -1
    assert lib.spmv_stream_copy(None, P(0x1008), 16, None) == -1


def test_version(lib):
    lib.spmv_version.restype = ctypes.c_char_p
    assert b"gfx950" in lib.spmv_version()
