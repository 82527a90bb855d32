"""SpMV throughput per storage format on one MI355X.

A step is one pass of the hot path over the resident matrix: y = A x in every
storage format the workload admits (CSR, ELLPACK-R, SELL-64, HYB, HEC; ELL-R is
refused where its padding exceeds the memory budget).  Conversions happen once
before timing (they are paid once per solve).  Inputs are already in HBM when
the timed region starts.

Reported per format: median apply time, GFLOP/s = 2 nnz / t, effective GB/s =
B_model / t with

    B_model = nnz (s_v + 4) + R_fmt + n s_v (y written) [+ n s_v if beta != 0]
              + n s_v (x read once)

(R_fmt = the format's row information), and that rate as a fraction of the
measured streaming copy (the library's copy kernel over 2 x 2 GiB) and of the
nominal 8 TB/s.  The CPU oracle (Dot2 CSR, OpenMP over the host cores) is
timed on the same matrix as a baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--dtype f64|f32] [--formats csr,hyb] [--no-cpu] [--cold]
Prints one JSON line.  Per format also: the rate on the CSR bytes model (one
byte count for every format); a matrix of under 1 MiB of values gets at least
1,000 timed applies per format; --cold adds medians of applies that each
follow a 1 GiB scratch read (nothing of the matrix or x left in the caches).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# launched by some applies only (SELL-64's chunk kernel and wide-slice beta pass)
OPTIONAL_KERNELS = {"k_sell_chunks", "k_sell_wide_beta"}
ALL_FORMATS = ["csr", "ellr", "sell64", "hyb", "hec"]
KERNELS = {
    "csr": "k_csr_vector",
    "ellr": "k_ell",
    "sell64": "k_sell (+ k_sell_chunks)",
    "hyb": "k_ell + k_tail<COO>",
    "hec": "k_ell + k_tail<CSR>",
}


def kernels_of(fmt: str, info: dict) -> str:
    """The kernels one apply of this handle launches."""
    if fmt == "csr":
        if info.get("csr_kernel") == "xblock":
            return "k_xblk"
        if info.get("csr_kernel") == "balanced":
            return "k_scale + k_tail%s<CSR>" % ("_win" if info["x_window"] else "")
        return _vector_kernel(info["subwave"], info["csr_rows"], info.get("csr_stage_slots", 0))
    k = KERNELS[fmt]
    if fmt in ("hyb", "hec") and info.get("tail_nnz", 1) == 0:
        k = "k_ell"
    if fmt in ("hyb", "hec") and info.get("tail_nnz", 1) > 0 and info.get("tail_kernel") == "xblock":
        k = k.replace("k_tail<CSR>", "k_xblk").replace("k_tail<COO>", "k_xblk")
    if fmt == "hec" and info.get("tail_kernel") == "vector":
        k = k.replace("k_tail<CSR>", _vector_kernel(info["tail_subwave"], info["tail_rows"],
                                                    info["tail_stage_slots"]))
    if fmt in ("ellr", "hyb", "hec") and info.get("x_window"):
        k = k.replace("k_ell", "k_ell_win").replace("k_tail", "k_tail_win")
    if fmt == "ellr" and info.get("ell_long_rows", 0) > 0:
        k += " + k_ell_long"  # the rows longer than the window kernel's head
    if fmt == "sell64" and info.get("x_window"):
        k = "(k_sell_wide_beta +) k_sell_win"
    return k


def _vector_kernel(sw: int, rows: int, slots: int) -> str:
    if slots > 0:
        return "k_csr_staged<S=%d>" % sw
    return "k_csr_vector<S=%d,R=%d>" % (sw, rows)


def row_info_bytes(fmt: str, n: int, tail_nnz: int = 0) -> int:
    """Bytes of row information an apply must read in each format."""
    if fmt == "csr":
        return 4 * (n + 1)
    if fmt == "ellr":
        return 4 * n
    if fmt == "sell64":
        ns = (n + 63) // 64
        return 4 * n + 4 * n + 8 * (ns + 1)       # lengths, permutation, slice starts
    if fmt == "hyb":
        return 4 * n + 4 * tail_nnz               # ELL lengths, COO row ids
    if fmt == "hec":
        return 4 * n + 4 * (n + 1)                # ELL lengths, tail row pointer
    raise ValueError(fmt)


def bytes_model(fmt: str, n: int, nnz: int, s_v: int, tail_nnz: int = 0,
                beta_nonzero: bool = False, x_alpha: float | None = None) -> float:
    """Algorithmic bytes of one apply.

    ``x_alpha`` is the fraction of x loads that reach memory per stored entry
    (alpha in the code balance of "Sparse matrix-vector multiplication on
    GPGPU clusters", Sect. 2.3); the default n / nnz is one pass over x.
    """
    xa = (n / nnz if nnz else 0.0) if x_alpha is None else x_alpha
    b = nnz * (s_v + 4) + row_info_bytes(fmt, n, tail_nnz) + n * s_v
    if beta_nonzero:
        b += n * s_v
    return b + xa * nnz * s_v


def _stream_handle(torch):
    return torch.cuda.current_stream()


def measure_stream_copy(torch, sf, gib: float = 2.0, reps: int = 20,
                        read_only: bool = False) -> float:
    """Median GB/s of the library's copy kernel over two 2 GiB buffers (or of
    its read-only stream over one)."""
    nbytes = int(gib * (1 << 30))
    src = torch.empty(nbytes // 8, dtype=torch.float64, device="cuda").fill_(1.0)
    dst = None if read_only else torch.empty_like(src)
    run = (lambda: sf.stream_read(src)) if read_only else (lambda: sf.stream_copy(dst, src))
    for _ in range(3):
        run()
    ts = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        run()
        e1.record()
        ts.append((e0, e1))
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in ts]))
    del src, dst
    torch.cuda.empty_cache()
    return (1 if read_only else 2) * nbytes / (ms * 1e-3) / 1e9


def cpu_baseline(a, x, s_v: int, target_s: float = 10.0, target_1core_s: float = 3.0,
                 nnz_1core: int = 25_000_000):
    """Time the CPU oracle (Dot2 CSR) on the full matrix over all host cores,
    and on one core over a contiguous block of rows holding about
    ``nnz_1core`` entries (a whole pass of a large matrix on one core would
    take most of a minute)."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    # one-core sample: the first rows up to about nnz_1core entries
    r1 = int(np.searchsorted(a.rowptr, min(nnz_1core, a.nnz), side="right")) - 1
    r1 = max(1, min(a.n, r1)) if a.n else 0
    rows1 = np.arange(r1, dtype=np.int64)
    nnz1 = int(a.rowptr[r1]) if a.n else 0

    def timed(threads, budget, rows):
        oracle.spmv(a, x, nthreads=threads, rows=rows)        # warm caches / threads
        reps, t = 0, 0.0
        t0 = time.perf_counter()
        while True:
            oracle.spmv(a, x, nthreads=threads, rows=rows)
            reps += 1
            t = time.perf_counter() - t0
            if t >= budget or reps >= 2000:
                return reps, t

    reps, t = timed(cores, target_s, None)
    reps1, t1 = timed(1, target_1core_s, rows1)
    bm = bytes_model("csr", a.n, a.nnz, s_v)
    bm1 = nnz1 * (s_v + 4) + 4 * (r1 + 1) + 2 * r1 * s_v
    return {"value": round(2.0 * a.nnz * reps / t / 1e9, 3), "unit": "GFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": "%d full applies of the same %d-row matrix (Dot2 fp64, OpenMP static "
                      "rows) in %.1f s; one core: rows 0..%d (%d entries) %d times in %.1f s"
                      % (reps, a.n, t, r1 - 1, nnz1, reps1, t1),
            "gbs_csr_model": round(bm * reps / t / 1e9, 2),
            "value_1core": round(2.0 * nnz1 * reps1 / t1 / 1e9, 3),
            "gbs_csr_model_1core": round(bm1 * reps1 / t1 / 1e9, 2)}


def kernel_bases(fmt: str, info: dict) -> set:
    """Base names of the kernels one apply of this handle launches (SELL's
    chunk kernel and wide-slice beta pass, present only with long slices, are
    left out)."""
    win = "_win" if info.get("x_window") else ""
    if fmt == "csr":
        if info.get("csr_kernel") == "xblock":
            return {"k_xblk"}
        if info.get("csr_kernel") == "balanced":
            return {"k_scale", "k_tail" + win}
        return {"k_csr_staged" if info.get("csr_stage_slots", 0) > 0 else "k_csr_vector"}
    if fmt == "sell64":
        return {"k_sell_win"} if info.get("x_window") else {"k_sell"}
    out = {"k_ell" + win}
    if fmt == "ellr" and info.get("ell_long_rows", 0) > 0:
        out.add("k_ell_long")
    if fmt in ("hyb", "hec") and info.get("tail_nnz", 0) > 0 and info.get("tail_kernel") == "xblock":
        out.add("k_xblk")
    elif fmt == "hec" and info.get("tail_nnz", 0) > 0 and info.get("tail_kernel") == "vector":
        out.add("k_csr_staged" if info.get("tail_stage_slots", 0) > 0 else "k_csr_vector")
    elif fmt in ("hyb", "hec") and info.get("tail_nnz", 0) > 0:
        out.add("k_tail" + win)
    return out


def traffic_for(key: str, bases: set, path: str | None = None):
    """HBM bytes of one apply from committed rocprofv3 counter runs
    (profiles/traffic.json), if the kernel sources have not changed since
    they were taken and the profiled apply ran the same kernels."""
    path = path or os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    recs = json.load(open(path)).get(key) or []
    for rec in recs if isinstance(recs, list) else [recs]:
        if {k.split("<")[0] for k in rec.get("kernels", [])} - OPTIONAL_KERNELS != bases:
            continue
        h = hashlib.sha256()
        for f in sorted(rec.get("sources", [])):
            h.update(open(os.path.join(ROOT, f), "rb").read())
        return rec.get("bytes_per_launch") if h.hexdigest() == rec.get("sha256") else None
    return None


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c5_fem_8m")
    ap.add_argument("--dtype", default="f64", choices=["f64", "f32"])
    ap.add_argument("--formats", default=",".join(ALL_FORMATS))
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-stream", action="store_true")
    ap.add_argument("--cold", action="store_true",
                    help="also time every format with a 1 GiB scratch read before each apply")
    ap.add_argument("--csr-kernel", default="auto", choices=["auto", "vector", "balanced", "xblock"],
                    help="CSR apply kernel (default: timed at conversion)")
    ap.add_argument("--no-graph", action="store_true",
                    help="time the whole steps eagerly instead of replaying a HIP graph of one")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU: this SpMV path runs on a single MI355X and has no "
              "multi-GPU mode (--gpus %d requested)" % args.gpus, file=sys.stderr)
        return 2

    import torch
    import gen
    import sparse_formats_amd as sf

    def log(m):
        print("[bench] " + m, file=sys.stderr, flush=True)

    npdt = np.float64 if args.dtype == "f64" else np.float32
    tdt = torch.float64 if args.dtype == "f64" else torch.float32
    s_v = 8 if args.dtype == "f64" else 4
    t0 = time.time()
    a, x_np, _, _ = gen.by_name(args.workload, npdt)
    log("workload %s: n=%d nnz=%d (generated in %.1fs)" % (args.workload, a.n, a.nnz,
                                                           time.time() - t0))
    rp = torch.from_numpy(a.rowptr).cuda()
    col = torch.from_numpy(a.col).cuda()
    val = torch.from_numpy(np.ascontiguousarray(a.val, npdt)).cuda()
    x = torch.from_numpy(x_np).cuda()
    y = torch.zeros(a.n, dtype=tdt, device="cuda")

    mats = {}
    setup_ms = {}
    refused = {}
    for fmt in args.formats.split(","):
        t1 = time.perf_counter()
        M = sf.Matrix.from_csr(rp, col, val, n=a.n)
        try:
            M.convert(fmt, csr_kernel=args.csr_kernel)
        except sf.SpmvError as e:
            refused[fmt] = str(e)
            M.close()
            log("%s refused: %s" % (fmt, e))
            continue
        torch.cuda.synchronize()
        setup_ms[fmt] = (time.perf_counter() - t1) * 1e3
        mats[fmt] = M
        log("%s built in %.0f ms: %s" % (fmt, setup_ms[fmt], M.info()))
    del rp, col, val
    torch.cuda.empty_cache()
    if not mats:
        log("every requested format was refused: %s" % refused)
        return 2

    stream_gbs = None if args.no_stream else measure_stream_copy(torch, sf)
    read_gbs = None if args.no_stream else measure_stream_copy(torch, sf, read_only=True)
    if stream_gbs:
        log("stream copy %.1f GB/s, read-only stream %.1f GB/s" % (stream_gbs, read_gbs))

    fmts = list(mats)
    for _ in range(args.warmup):
        for f in fmts:
            mats[f].apply(y, x)
    torch.cuda.synchronize()
    ev = {f: [] for f in fmts}
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        for f in fmts:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            mats[f].apply(y, x)
            e1.record()
            ev[f].append((e0, e1))
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    # a launch-bound matrix (a few hundred KB) gets at least 1,000 timed
    # applies per format for its medians
    reps = args.steps if a.nnz * s_v >= (1 << 20) else max(args.steps, 1000)
    for f in fmts:
        for _ in range(reps - args.steps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            mats[f].apply(y, x)
            e1.record()
            ev[f].append((e0, e1))
    torch.cuda.synchronize()
    # cold: reading 1 GiB of scratch through the caches before each apply
    # empties the Infinity Cache of the matrix and x (a read leaves no dirty
    # lines, so the apply pays for no write-backs of the flush; the library's
    # read stream would not do: its nontemporal loads leave the caches as
    # they are).  Only the apply is timed.
    cold = {f: [] for f in fmts} if args.cold else None
    if args.cold:
        scratch = torch.ones(1 << 27, dtype=torch.float64, device="cuda")
        for f in fmts:
            for r in range(args.steps):
                scratch.sum()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                mats[f].apply(y, x)
                e1.record()
                cold[f].append((e0, e1))
        torch.cuda.synchronize()
        del scratch
        torch.cuda.empty_cache()
    step_timing = "eager"
    if not args.no_graph:
        # the step rate without host launch gaps: the same applies, captured
        # once as a HIP graph of one step and replayed
        cur = torch.cuda.current_stream()
        side = torch.cuda.Stream()
        side.wait_stream(cur)
        with torch.cuda.stream(side):
            for f in fmts:
                mats[f].apply(y, x)
        cur.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for f in fmts:
                mats[f].apply(y, x)
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        eager_ms = total_ms
        start.record()
        for _ in range(args.steps):
            graph.replay()
        end.record()
        torch.cuda.synchronize()
        total_ms = start.elapsed_time(end)
        step_timing = "hip_graph (eager steps: %.5f ms)" % (eager_ms / args.steps)
        del graph

    per = {}
    mats_info = {f: mats[f].info() for f in fmts}
    bm_csr = bytes_model("csr", a.n, a.nnz, s_v)  # one byte count for every format
    for f in fmts:
        ts = np.array([e0.elapsed_time(e1) for e0, e1 in ev[f]])
        med = float(np.median(ts))
        info = mats_info[f]
        bm = bytes_model(f, a.n, a.nnz, s_v, info["tail_nnz"])
        gbs = bm / (med * 1e-3) / 1e9
        per[f] = {
            "ms_median": round(med, 5), "ms_min": round(float(ts.min()), 5),
            "ms_p90": round(float(np.percentile(ts, 90)), 5), "timed_applies": int(ts.size),
            "gflops": round(2 * a.nnz / (med * 1e-3) / 1e9, 2),
            "eff_gbs": round(gbs, 1), "bytes_model": int(bm),
            "eff_gbs_csr_model": round(bm_csr / (med * 1e-3) / 1e9, 1),
            "frac_stream": round(gbs / stream_gbs, 4) if stream_gbs else None,
            "frac_stream_csr_model": (round(bm_csr / (med * 1e-3) / 1e9 / stream_gbs, 4)
                                      if stream_gbs else None),
            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "slots": info["slots"], "ell_width": info["ell_width"],
            "tail_nnz": info["tail_nnz"], "setup_ms": round(setup_ms[f], 1),
            "kernels": kernels_of(f, info), "x_window": info["x_window"],
        }
        if cold is not None:
            tc = float(np.median([e0.elapsed_time(e1) for e0, e1 in cold[f]]))
            per[f]["cold_ms_median"] = round(tc, 5)
            per[f]["cold_frac_stream"] = (round(bm / (tc * 1e-3) / 1e9 / stream_gbs, 4)
                                          if stream_gbs else None)
    # best format: the shortest apply (the same ranking as GFLOP/s and as the
    # CSR bytes model, one byte count for every format)
    best = min(per, key=lambda f: per[f]["ms_median"])
    dom = max(per, key=lambda f: per[f]["ms_median"])

    def roof(f):
        d = per[f]
        achieved = d["bytes_model"] / (d["ms_median"] * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic_for("%s:%s:%s" % (args.workload, args.dtype, f),
                                       kernel_bases(f, mats_info[f])),
                "kernel": "%s apply (%s)" % (f, d["kernels"]),
                "frac_of_stream": d["frac_stream"],
                "frac_of_read_stream": round(achieved / read_gbs, 4) if read_gbs else None}

    roofline = roof(dom)
    flops_step = 2.0 * a.nnz * len(fmts)
    out = {
        "metric": "SpMV GFLOP/s and effective HBM GB/s (% of roofline) per format, " + args.dtype,
        "value": round(flops_step * args.steps / (total_ms * 1e-3) / 1e9, 2),
        "unit": "GFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": args.dtype, "data": "synthetic",
        "config": {"workload": args.workload, "n": a.n, "nnz": a.nnz,
                   "formats": fmts, "refused": refused,
                   "step": "one apply y = A x in each listed format",
                   "step_timing": step_timing,
                   "value": "2 nnz x formats per step / step time"},
        "best_format": {"format": best, "ranking": "shortest apply (= highest GFLOP/s "
                                                   "and CSR-bytes-model rate)",
                        "gflops": per[best]["gflops"],
                        "eff_gbs": per[best]["eff_gbs"],
                        "frac_stream": per[best]["frac_stream"],
                        "eff_gbs_csr_model": per[best]["eff_gbs_csr_model"],
                        "frac_stream_csr_model": per[best]["frac_stream_csr_model"]},
        "stream_copy_gbs": round(stream_gbs, 1) if stream_gbs else None,
        "stream_read_gbs": round(read_gbs, 1) if read_gbs else None,
        "formats": per,
        "roofline": roofline,
        "roofline_best": roof(best),
    }
    if not args.no_cpu:
        log("timing the CPU oracle ...")
        out["cpu_baseline"] = cpu_baseline(a, x_np, s_v)
    for M in mats.values():
        M.close()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
