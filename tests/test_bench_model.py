"""The benchmark's bytes model, pinned by the pages' PCIe thresholds and by
hand-computed byte counts, plus the shape of the bench JSON line."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

GOLD = os.path.join(os.path.dirname(__file__), "golden", "p1_pcie_thresholds.txt")


def threshold(alpha_kind, ratio, penalty):
    """N_nzr at which device spMVM time equals (50 %) or is 10x (10 %) the
    PCIe time of moving RHS in and LHS out (16 bytes per row, DP).

    Device time per row = bytes_model per row / B_GPU for an ELL-R matrix with
    N_nzr entries per row; PCIe time per row = 16 / B_PCI.
    """
    def dev_bytes_per_row(nnzr):
        n = 1000
        alpha = 1.0 / nnzr if alpha_kind == "inv" else 1.0
        return bench.bytes_model("ellr", n, int(n * nnzr), 8, x_alpha=alpha) / n

    target = 16.0 * ratio * (1 if penalty == 50 else 10)
    lo, hi = 0.01, 1e4
    for _ in range(200):
        mid = (lo + hi) / 2
        if dev_bytes_per_row(mid) < target:
            lo = mid
        else:
            hi = mid
    return lo


def test_pcie_thresholds_from_code_balance():
    """[GPGPU clusters] Sect. 2.3 prints 25, 7, 80, 266; the reconstructed
    code balance (8 + 4 + 8 alpha per entry, 4 + 8 per row) gives them
    within one."""
    for line in open(GOLD):
        if line.startswith("#") or not line.strip():
            continue
        _, kind, ratio, penalty, page = line.split()
        got = threshold(kind, float(ratio), int(penalty))
        assert abs(got - float(page)) <= 1.0, (kind, ratio, penalty, got, page)


def test_bytes_model_exact_counts():
    # C1: 20,224 entries, 4,096 rows, fp64, CSR: 12*20224 + 4*4097 + 8*4096 + 8*4096
    assert bench.bytes_model("csr", 4096, 20224, 8) == 12 * 20224 + 4 * 4097 + 16 * 4096
    assert bench.bytes_model("csr", 4096, 20224, 8) == 324_612
    # C3: 55,742,968 entries on 2,097,152 rows
    assert bench.bytes_model("csr", 2_097_152, 55_742_968, 8) == 710_858_660
    assert bench.bytes_model("csr", 2_097_152, 55_742_968, 4) == 471_109_572
    # beta != 0 reads y once more
    assert bench.bytes_model("ellr", 100, 1000, 8, beta_nonzero=True) == \
        bench.bytes_model("ellr", 100, 1000, 8) + 800
    # per-format row information
    assert bench.row_info_bytes("hyb", 10, tail_nnz=7) == 40 + 28
    assert bench.row_info_bytes("hec", 10) == 40 + 44
    assert bench.row_info_bytes("sell64", 130) == 4 * 130 * 2 + 8 * 4


def test_gpus_above_one_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


@pytest.mark.gpu
def test_bench_json_line():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload",
                        "c1_laplace2d_64", "--steps", "3", "--warmup", "1", "--no-cpu",
                        "--no-stream"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    out = json.loads(r.stdout.strip().splitlines()[-1])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "formats", "best_format"):
        assert k in out, k
    assert out["config"]["workload"] == "c1_laplace2d_64"
    assert set(out["formats"]) == {"csr", "ellr", "sell64", "hyb", "hec"}
    assert out["config"]["step_timing"].startswith("hip_graph")
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in out["roofline"]


def test_traffic_record_checks(tmp_path):
    """The bench reports counter traffic only for the kernels it launched and
    only while their sources are unchanged."""
    import hashlib
    srcs = ["sparse_formats_amd/csrc/k_tail.hip", "sparse_formats_amd/csrc/common.h"]
    h = hashlib.sha256()
    for f in sorted(srcs):
        h.update(open(os.path.join(ROOT, f), "rb").read())
    rec = {"w:f64:csr": [{"kernels": ["k_scale<double>", "k_tail<double, false>"],
                          "bytes_per_launch": 123, "sources": srcs, "sha256": h.hexdigest()},
                         {"kernels": ["k_csr_vector<double, 8, 1>"], "bytes_per_launch": 99,
                          "sources": srcs, "sha256": h.hexdigest()}],
           "w:f64:hyb": {"kernels": ["k_ell<double>", "k_tail<double, true>"],
                         "bytes_per_launch": 7, "sources": srcs, "sha256": "0" * 64}}
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(rec))
    bal = bench.kernel_bases("csr", {"csr_kernel": "balanced", "x_window": 0})
    assert bal == {"k_scale", "k_tail"}
    assert bench.traffic_for("w:f64:csr", bal, str(p)) == 123
    vec = bench.kernel_bases("csr", {"csr_kernel": "vector", "x_window": 0})
    assert bench.traffic_for("w:f64:csr", vec, str(p)) == 99            # the other record
    win = bench.kernel_bases("csr", {"csr_kernel": "balanced", "x_window": 1})
    assert bench.traffic_for("w:f64:csr", win, str(p)) is None          # window variant
    hyb = bench.kernel_bases("hyb", {"x_window": 0, "tail_nnz": 5})
    assert bench.traffic_for("w:f64:hyb", hyb, str(p)) is None          # stale sources
    assert bench.traffic_for("w:f64:hec", hyb, str(p)) is None          # no record
    assert bench.kernel_bases("hec", {"x_window": 1, "tail_nnz": 0}) == {"k_ell_win"}
    staged = bench.kernel_bases("csr", {"csr_kernel": "vector", "x_window": 0,
                                        "csr_stage_slots": 512})
    assert staged == {"k_csr_staged"}
    assert bench.traffic_for("w:f64:csr", staged, str(p)) is None       # no staged record
    hec_vec = {"x_window": 0, "tail_nnz": 9, "tail_kernel": "vector", "tail_subwave": 2,
               "tail_rows": 1, "tail_stage_slots": 256}
    assert bench.kernel_bases("hec", hec_vec) == {"k_ell", "k_csr_staged"}
    assert bench.kernels_of("hec", hec_vec) == "k_ell + k_csr_staged<S=2>"
    hec_vec.update(tail_stage_slots=0, tail_subwave=4, tail_rows=2)
    assert bench.kernel_bases("hec", hec_vec) == {"k_ell", "k_csr_vector"}
    assert bench.kernels_of("hec", hec_vec) == "k_ell + k_csr_vector<S=4,R=2>"
    assert bench.kernels_of("hyb", {"x_window": 1, "tail_nnz": 0}) == "k_ell_win"
    assert bench.kernels_of("hyb", {"x_window": 0, "tail_nnz": 3}) == "k_ell + k_tail<COO>"
    # HYB / HEC tails by column slices
    for fmt in ("hyb", "hec"):
        t = {"x_window": 1, "tail_nnz": 3, "tail_kernel": "xblock"}
        assert bench.kernels_of(fmt, t) == "k_ell_win + k_xblk"
        assert bench.kernel_bases(fmt, t) == {"k_ell_win", "k_xblk"}
    # the column-slice CSR kernel and its traffic record
    xb = {"csr_kernel": "xblock", "x_window": 0, "subwave": 1, "csr_rows": 1}
    assert bench.kernel_bases("csr", xb) == {"k_xblk"}
    assert bench.kernels_of("csr", xb) == "k_xblk"
    rec["w:f64:csr"][0]["kernels"] = ["k_scale<double>", "k_tail_win<double, false>"]
    rec["w:f64:csr"].append({"kernels": ["k_xblk<double>"],
                             "bytes_per_launch": 55, "sources": srcs, "sha256": h.hexdigest()})
    p.write_text(json.dumps(rec))
    assert bench.traffic_for("w:f64:csr", bench.kernel_bases("csr", xb), str(p)) == 55


def test_counter_summary(tmp_path, monkeypatch):
    """profile_summary.py counters: the counters of the last dispatch of each
    kernel of the last apply, with several counter rows per dispatch."""
    import profile_summary as ps
    out = tmp_path / "pmc"
    d = out / "PMC1_w_csr-balanced"
    d.mkdir(parents=True)
    (out / "PMC1_w_csr-balanced.txt").write_text("A B\n")
    rows = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value"]
    disp = 0
    for rep in range(3):       # three applies, then the last one is kept
        for k in ("spmv::k_scale<double>(x)", "spmv::k_tail<double, false>(x)"):
            disp += 1
            for c in ("A", "B"):
                rows.append('%d,"%s",%s,%d' % (disp, k, c, 10 * rep + (c == "B")))
    (d / "run_counter_collection.csv").write_text("\n".join(rows) + "\n")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(ps, "ROOT", str(tmp_path))
    monkeypatch.setattr(sys, "argv", ["x", "counters", str(out), "w", "csr-balanced"])
    ps.counters_main()
    text = (tmp_path / "profiles" / "spmv_w_f64_csr-balanced_counters.md").read_text()
    body = [l for l in text.splitlines() if l.startswith("| k_")]
    assert [l.split(" | ")[0] for l in body] == ["| k_scale<double>", "| k_tail<double, false>"]
    assert all(l.endswith("| 20 | 21 |") for l in body)      # the last apply's values
    assert "--formats csr --csr-kernel balanced" in text


def _trace(names):
    """rocprofv3 kernel-trace rows: dispatch i runs 10 * (i + 1) us."""
    rows, t = [], 0
    for i, k in enumerate(names):
        d = 10_000 * (i + 1)
        rows.append({"Kernel_Name": "void spmv::%s(int)" % k, "Start_Timestamp": str(t),
                     "End_Timestamp": str(t + d)})
        t += d + 1000
    return rows


C4_KERNELS = {"csr": "k_xblk", "sell64": "k_sell (+ k_sell_chunks)",
              "hyb": "k_ell + k_tail<COO>", "hec": "k_ell + k_tail<CSR>"}
C4_STEP = ["k_xblk<double>", "k_sell<double, true>",
           "k_sell_chunks<double, true>", "k_ell<double, true>", "k_tail<double, true>",
           "k_ell<double, true>", "k_tail<double, false>"]


def test_profile_attribution_c4_step_with_stray_dispatch():
    """Each format gets its own kernels: the column-slice CSR apply, SELL with
    its chunk kernel, HYB's COO and HEC's CSR tail; a stray
    dispatch before the first step is skipped, not counted as an apply."""
    import profile_summary as ps
    fmts = ["csr", "sell64", "hyb", "hec"]
    trace = _trace(["k_tail<double, false>"] + C4_STEP * 3)
    out = ps.per_format_applies(trace, fmts, C4_KERNELS)
    assert [len(out[f]) for f in fmts] == [3, 3, 3, 3]
    assert out["csr"][0][0] == "k_xblk<double>"
    assert out["sell64"][0][0] == "k_sell<double, true> + k_sell_chunks<double, true>"
    assert out["hyb"][0][0] == "k_ell<double, true> + k_tail<double, true>"
    assert out["hec"][0][0] == "k_ell<double, true> + k_tail<double, false>"
    # durations: dispatch i takes 10 (i + 1) us; the stray one is dispatch 0
    assert out["csr"][0][1] == 20 and out["hec"][0][1] == 70 + 80


def test_profile_attribution_trace_from_mid_step():
    """A trace that begins inside a step (here at HYB's apply) is attributed
    from its first whole apply on; the half apply before it is dropped."""
    import profile_summary as ps
    fmts = ["csr", "sell64", "hyb", "hec"]
    trace = _trace(["k_sell_chunks<double, true>"] + C4_STEP[3:] + C4_STEP * 2)
    out = ps.per_format_applies(trace, fmts, C4_KERNELS)
    assert [len(out[f]) for f in fmts] == [2, 2, 3, 3]
    assert all(k == "k_ell<double, true> + k_tail<double, true>" for k, _ in out["hyb"])
    assert all(k == "k_xblk<double>" for k, _ in out["csr"])
    # the C3 case: ELL-R, HYB and HEC all launch k_ell alone; step order decides
    c3 = {"csr": "k_csr_staged<S=4>", "ellr": "k_ell", "sell64": "k_sell (+ k_sell_chunks)",
          "hyb": "k_ell", "hec": "k_ell"}
    f5 = list(c3)
    step = ["k_csr_staged<double, 4>", "k_ell<double, true>", "k_sell<double, true>",
            "k_ell<double, true>", "k_ell<double, true>"]
    out = ps.per_format_applies(_trace(step * 2), f5, c3)
    assert [len(out[f]) for f in f5] == [2] * 5
    assert out["csr"][0][0] == "k_csr_staged<double, 4>"
    assert out["hec"][1][1] == 100


def test_profile_attribution_sell_window():
    """SELL-64 with the LDS window: its apply is k_sell_win, preceded by the
    beta pass over the wide slices when the matrix has some; both variants are
    one apply, and the bench names the kernels and traffic bases alike."""
    import profile_summary as ps
    info = {"x_window": 1}
    assert bench.kernels_of("sell64", info) == "(k_sell_wide_beta +) k_sell_win"
    assert bench.kernel_bases("sell64", info) == {"k_sell_win"}
    assert bench.kernel_bases("sell64", {"x_window": 0}) == {"k_sell"}
    kern = {"csr": "k_scale + k_tail_win<CSR>", "sell64": bench.kernels_of("sell64", info),
            "hyb": "k_ell_win + k_tail_win<COO>"}
    fmts = list(kern)
    step_wide = ["k_scale<double>", "k_tail_win<double, false>", "k_sell_wide_beta<double>",
                 "k_sell_win<double, true>", "k_ell_win<double, true>", "k_tail_win<double, true>"]
    step_plain = ["k_scale<double>", "k_tail_win<double, false>", "k_sell_win<double, true>",
                  "k_ell_win<double, true>", "k_tail_win<double, true>"]
    out = ps.per_format_applies(_trace(step_wide + step_plain), fmts, kern)
    assert [len(out[f]) for f in fmts] == [2, 2, 2]
    assert out["sell64"][0][0] == "k_sell_wide_beta<double> + k_sell_win<double, true>"
    assert out["sell64"][1][0] == "k_sell_win<double, true>"
    assert out["sell64"][0][1] == 30 + 40     # dispatches 2 and 3 (10 (i + 1) us)
    # the counter summary's last apply of a SELL-window run
    seq = [("k_sell_wide_beta", "k_sell_wide_beta<double>"), ("k_sell_win", "k_sell_win<double, true>")]
    assert ps.split_apply([("k_copy", "k_copy")] + seq) == seq
    with pytest.raises(AssertionError):
        ps.split_apply([("k_copy", "k_copy")])


def test_profile_attribution_ell_window_long_rows():
    """ELL-R with the LDS window and a few long rows: the window kernel takes
    every row's head, then k_ell_long the long rows' rest; one apply of two
    kernels, named alike by the bench and the profile summary (the FEM block's
    step: column-slice CSR, ELL-R, SELL-64, HYB, HEC)."""
    import profile_summary as ps
    info = {"x_window": 1, "ell_long_rows": 80000, "ell_head": 40}
    assert bench.kernels_of("ellr", info) == "k_ell_win + k_ell_long"
    assert bench.kernel_bases("ellr", info) == {"k_ell_win", "k_ell_long"}
    assert bench.kernels_of("ellr", {"x_window": 1, "ell_long_rows": 0}) == "k_ell_win"
    c5 = {"csr": "k_xblk", "ellr": "k_ell_win + k_ell_long",
          "sell64": "(k_sell_wide_beta +) k_sell_win", "hyb": "k_ell_win + k_tail_win<COO>",
          "hec": "k_ell_win + k_tail_win<CSR>"}
    f5 = list(c5)
    step = ["k_xblk<double, 8>", "k_ell_win<double, true, true>", "k_ell_long<double, true>",
            "k_sell_wide_beta<double>", "k_sell_win<double, true>",
            "k_ell_win<double, true, false>", "k_tail_win<double, true>",
            "k_ell_win<double, true, false>", "k_tail_win<double, false>"]
    out = ps.per_format_applies(_trace(step * 3), f5, c5)
    assert [len(out[f]) for f in f5] == [3] * 5
    assert out["ellr"][0][0] == "k_ell_win<double, true, true> + k_ell_long<double, true>"
    assert out["hyb"][2][0] == "k_ell_win<double, true, false> + k_tail_win<double, true>"
    # durations: dispatch i takes 10 (i + 1) us, the step's second apply is dispatches 1-2
    assert out["ellr"][0][1] == 20 + 30
