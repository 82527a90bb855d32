"""The oracle's pins catch plausible mistakes: each case below plants one
mistake in a copy of oracle.c (a dropped term, a wrong sign, index or bound,
a transposed layout, a reversed sort key, a wrong rule), builds it with the
oracle's own flags, and runs the pin suites (tests/test_oracle_*.py) against
it in a child process; at least one pin must fail.  Nothing here touches a
GPU or the HIP library."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PIN_SUITES = ["tests/test_oracle_pins.py", "tests/test_oracle_converters.py",
              "tests/test_oracle_solvers.py"]

# (name, text in oracle.c, replacement)
PLANTED = [
    ("dot2_drops_correction", "    return s + c;\n}", "    return s;\n}"),
    ("twosum_wrong_sign", "*e = (a - (x - z)) + (b - z);", "*e = (a - (x - z)) - (b - z);"),
    ("twoprod_drops_error", "*e = fma(a, b, -x);", "*e = 0.0;"),
    ("row_drops_last_entry", "for (int64_t k = k0; k < k1; ++k) {",
     "for (int64_t k = k0; k < k1 - 1; ++k) {"),
    ("x_index_shifted", "two_prod(val[k], x[col[k]], &p, &ep);",
     "two_prod(val[k], x[col[k] > 0 ? col[k] - 1 : 0], &p, &ep);"),
    ("beta_term_dropped", "            yv = alpha * r + by;", "            yv = alpha * r;"),
    ("alpha_scales_beta_term", "            yv = alpha * r + by;", "            yv = alpha * (r + by);"),
    ("scale_misses_beta", "            sc += fabs(by);", "            sc += 0.0;"),
    ("ell_slot_row_major", "int64_t slot = (p / B) * W * B + j * B + p % B;",
     "int64_t slot = (p / B) * W * B + (p % B) * W + j;"),
    ("sell_sort_ascending", "    int64_t lb = g_rowptr[b + 1] - g_rowptr[b];\n    if (la != lb)\n"
     "        return la > lb ? -1 : 1;",
     "    int64_t lb = g_rowptr[b + 1] - g_rowptr[b];\n    if (la != lb)\n"
     "        return la < lb ? -1 : 1;"),
    ("sell_width_first_row", "            if (len_sorted[r] > w)", "            if (r == 64 * s)"),
    ("sell_slot_transposed", "int64_t slot = slice_ptr[r / 64] + 64 * j + r % 64;",
     "int64_t slot = slice_ptr[r / 64] + j + (r % 64) * (len > 0 ? len : 1);"),
    ("permuted_basis_inverse_wrong", "            inv[perm[r]] = r;", "            inv[r] = perm[r];"),
    ("width_rule_strict", "        if (cnt >= need)", "        if (cnt > need)"),
    ("regular_width_strict", "        if (100 * longer <= n)", "        if (100 * longer < n)"),
    ("tail_skips_one", "for (int64_t k = rowptr[i] + K; k < rowptr[i + 1]; ++k) {",
     "for (int64_t k = rowptr[i] + K + 1; k < rowptr[i + 1]; ++k) {"),
    ("cg_beta_inverted", "        double beta = rr_new / rr;", "        double beta = rr / rr_new;"),
    ("bicgstab_omega_sign", "            r[i] = s[i] - omega * t[i];", "            r[i] = s[i] + omega * t[i];"),
]


def _build(tmp_path, text):
    src = tmp_path / "planted.c"
    src.write_text(text)
    so = tmp_path / "libplanted.so"
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC",
           "-o", str(so), str(src), "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return so


@pytest.mark.parametrize("name,old,new", PLANTED, ids=[p[0] for p in PLANTED])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, "the planted text must match exactly one place: %s" % name
    so = _build(tmp_path, text.replace(old, new))
    env = dict(os.environ, ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", *PIN_SUITES], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode != 0, "no pin caught the planted mistake %s:\n%s" % (name, r.stdout[-2000:])


def test_unmodified_copy_passes(tmp_path):
    """The harness itself: the same build of the unmodified source passes."""
    so = _build(tmp_path, open(SRC).read())
    env = dict(os.environ, ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", *PIN_SUITES], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:]
