"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (signed
overflow and other undefined behaviour abort the run):

* the kernels' index arithmetic (sparse_formats_amd/csrc/index_math.h, the
  functions the kernels call) at the 2^31 / 2^32 boundaries and against plain
  definitions (tests/host/index_math_test.cpp);
* the oracle (oracle/oracle.c) under its own pin suites;
* the library's host code (api.hip with -Xarch_host sanitizers, linked with
  the kernel objects of the last build) under the C-ABI argument tests, which
  run without a GPU.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _preload():
    libs = []
    for name in ("libasan.so", "libubsan.so"):
        p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True,
                           text=True).stdout.strip()
        if not os.path.isabs(p):
            pytest.skip("gcc has no %s" % name)
        libs.append(p)
    return ":".join(libs)


def _clang_asan_runtime():
    """The shared AddressSanitizer runtime of ROCm's clang (hipcc's host
    sanitizers need clang's runtime, not gcc's)."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/*/libclang_rt.asan-x86_64.so"))
    if not hits:
        pytest.skip("no clang AddressSanitizer runtime under /opt/rocm")
    return hits[-1]


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, "%s\n%s%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r.stdout


def test_index_math_under_sanitizers(tmp_path):
    exe = str(tmp_path / "index_math_test")
    _run(["g++", "-O1", "-g", "-std=c++17", *SAN, "-I/opt/rocm/include",
          "-D__HIP_PLATFORM_AMD__", os.path.join(ROOT, "tests", "host", "index_math_test.cpp"),
          "-o", exe])
    out = _run([exe])
    assert "checks passed" in out


def test_oracle_under_sanitizers(tmp_path):
    so = str(tmp_path / "liboracle_san.so")
    _run(["gcc", "-O1", "-g", *SAN, "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
          "-shared", "-fPIC", os.path.join(ROOT, "oracle", "oracle.c"), "-o", so, "-lm"])
    env = dict(os.environ, ORACLE_LIB=so, LD_PRELOAD=_preload(),
               ASAN_OPTIONS="detect_leaks=0")
    out = _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                os.path.join(ROOT, "tests", "test_oracle_converters.py"),
                os.path.join(ROOT, "tests", "test_oracle_solvers.py")], env=env)
    assert " passed" in out and "failed" not in out


def test_library_host_code_under_sanitizers(tmp_path):
    bdir = os.path.join(ROOT, "sparse_formats_amd", "csrc", "_build")
    others = [os.path.join(bdir, f + ".o") for f in ("k_csr", "k_ell", "k_tail", "k_vec", "k_xblk")]
    if not all(os.path.exists(o) for o in others):
        pytest.skip("kernel objects not built (run __graft_entry__.build() first)")
    obj = str(tmp_path / "api_san.o")
    so = str(tmp_path / "libspmv_san.so")
    # host-side sanitizers only: each -fsanitize applies to the host pass
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-munsafe-fp-atomics",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=all",
          "-I" + os.path.join(ROOT, "include"),
          "-c", os.path.join(ROOT, "sparse_formats_amd", "csrc", "api.hip"), "-o", obj])
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host",
          "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host",
          "-shared-libsan", "-o", so, obj, *others])
    rt = _clang_asan_runtime()
    env = dict(os.environ, SPMV_ABI_LIB=so, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0",
               LD_LIBRARY_PATH=os.path.dirname(rt) + ":" + os.environ.get("LD_LIBRARY_PATH", ""))
    out = _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                os.path.join(ROOT, "tests", "test_abi_cpu.py")], env=env)
    assert " passed" in out and "failed" not in out
