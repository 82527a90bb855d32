"""Summaries of the rocprofv3 runs behind the benchmark's roofline figures.

Reads the output directories of the runs made by these commands (from the
repository root on the MI355X machine, W the workload):

    rocprofv3 --kernel-trace --stats --output-format csv -d <out>/stats_W -o run \
        -- python3 bench.py --workload W --steps 10 --warmup 2 --no-cpu
    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/FETCH_SIZE_W_F -o run \
        -- python3 bench.py --workload W --formats F --steps 2 --warmup 1 --no-cpu
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/WRITE_SIZE_W_F -o run \
        -- python3 bench.py --workload W --formats F --steps 2 --warmup 1 --no-cpu

(for CSR once per kernel: F = csr-vector / csr-balanced / csr-xblock with
--formats csr --csr-kernel vector / balanced / xblock)

and writes profiles/spmv_<W>_<dtype>_kernel_stats.md, ..._fetch_write.md and the
per-apply HBM bytes of every format into profiles/traffic.json (keyed by
workload:dtype:format, with a hash of the kernel sources so that the bench
drops the figure once a kernel changes).

Usage: python profile_summary.py <out> <workload> [dtype]
       python profile_summary.py counters <out> <workload> <format> [dtype]

The second form summarizes counter passes of one format (each pass a
directory <out>/PMC<k>_<workload>_<format> made by
    rocprofv3 --pmc <counters> --output-format csv -d <dir> -o run \
        -- python3 bench.py --workload W --formats F [--csr-kernel K] --steps 2 --warmup 1 --no-cpu
with the counters listed in <dir>.txt) into
profiles/spmv_<W>_<dtype>_<format>_counters.md: the counters of the last
dispatch of every kernel of the apply.
"""
import csv
import hashlib
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
FORMATS = ["csr-vector", "csr-balanced", "csr-xblock", "ellr", "sell64", "hyb", "hec"]
APPLY = ("k_csr_vector", "k_csr_staged", "k_scale", "k_tail", "k_tail_win", "k_ell", "k_ell_win", "k_sell",
         "k_sell_chunks", "k_sell_win", "k_sell_wide_beta", "k_xblk", "k_ell_long")
# kernels an apply launches only for some matrices: SELL-64's chunk kernel
# after k_sell, and its beta pass over the wide slices before k_sell_win
OPTIONAL_AFTER = {"k_sell": "k_sell_chunks"}
OPTIONAL_BEFORE = {"k_sell_win": "k_sell_wide_beta"}
SOURCES = ["sparse_formats_amd/csrc/" + f for f in
           ("api.hip", "k_csr.hip", "k_ell.hip", "k_tail.hip", "k_xblk.hip", "common.h", "internal.h",
            "index_math.h")]


def short(name):
    n = name.replace("(anonymous namespace)::", "").replace("spmv::", "")
    n = n[5:] if n.startswith("void ") else n
    base = n.split("(")[0]
    return base.split("<")[0], base


def source_hash():
    h = hashlib.sha256()
    for f in sorted(SOURCES):
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()


def rows_of(d, suffix):
    f = [x for x in os.listdir(d) if x.endswith(suffix)][0]
    return list(csv.DictReader(open(os.path.join(d, f))))


def split_apply(seq):
    """Split a format's last apply off the end of a dispatch list [(short, full)]."""
    out = []
    seen = set()
    for s, full in reversed(seq):
        if s not in APPLY or full in seen:
            break
        # an apply launches at most one ELL, one tail, one scale, one SELL kernel
        seen.add(full)
        out.append((s, full))
    assert out, "the run ends with no apply kernel (last: %s)" % (seq[-1:] or "none")
    return list(reversed(out))


def signature(kernels):
    """[(base name, COO tail?)] of one apply from the bench's kernel string of a
    format (e.g. "k_ell_win + k_tail_win<COO>", "k_xblk"); SELL's
    optional kernels (in parentheses) are left out."""
    sig = []
    for part in kernels.replace("(+ k_sell_chunks)", "").replace("(k_sell_wide_beta +)",
                                                                 "").split("+"):
        part = part.strip()
        if part:
            coo = True if "<COO>" in part else False if "<CSR>" in part else None
            sig.append((part.split("<")[0], coo))
    return sig


def _matches(disp, entry):
    base, coo = entry
    if disp[0] != base:
        return False
    return coo is None or disp[1].endswith("true>" if coo else "false>")


def per_format_applies(timed, formats, kernels):
    """Attribute the bench's apply dispatches to formats.  `kernels` maps each
    format to the bench line's kernel string for it; every step applies the
    formats in order.  At each dispatch the next format of the step is tried
    first, then the others (a trace may begin inside a step); a dispatch that
    starts no format's apply is skipped.  SELL-64's chunk kernel joins its
    apply when it follows."""
    out = {f: [] for f in formats}
    sigs = {f: signature(kernels[f]) for f in formats}
    names = [(short(r["Kernel_Name"])[0], short(r["Kernel_Name"])[1],
              (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3) for r in timed]

    def match_at(i, f):
        sig = sigs[f]
        return i + len(sig) <= len(names) and all(
            _matches(names[i + j], sig[j]) for j in range(len(sig)))

    def match_with_prefix(i, f):
        """Length of the optional kernel before f's apply at i (0 or 1), or None."""
        if match_at(i, f):
            return 0
        first = sigs[f][0][0] if sigs[f] else None
        if (i < len(names) and first in OPTIONAL_BEFORE
                and names[i][0] == OPTIONAL_BEFORE[first] and match_at(i + 1, f)):
            return 1
        return None

    i, k = 0, 0
    while i < len(names):
        order = [formats[(k + d) % len(formats)] for d in range(len(formats))]
        f = next((g for g in order if match_with_prefix(i, g) is not None), None)
        if f is None:
            i += 1
            continue
        m = len(sigs[f]) + match_with_prefix(i, f)
        ks = [n[1] for n in names[i:i + m]]
        tot = sum(n[2] for n in names[i:i + m])
        i += m
        last = sigs[f][-1][0] if sigs[f] else None
        if last in OPTIONAL_AFTER and i < len(names) and names[i][0] == OPTIONAL_AFTER[last]:
            ks.append(names[i][1])
            tot += names[i][2]
            i += 1
        out[f].append((" + ".join(ks), tot))
        k = (formats.index(f) + 1) % len(formats)
    return out


def main():
    out_dir, workload = sys.argv[1], sys.argv[2]
    dtype = sys.argv[3] if len(sys.argv) > 3 else "f64"
    tag = "%s_%s" % (workload, dtype)
    dt_flag = "" if dtype == "f64" else " --dtype " + dtype
    # ---- kernel statistics of the default bench
    sd = os.path.join(out_dir, "stats_" + workload)
    stats = rows_of(sd, "kernel_stats.csv")
    trace = sorted(rows_of(sd, "kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"]))
    last_copy = max(i for i, r in enumerate(trace) if short(r["Kernel_Name"])[0] == "k_copy")
    timed = [r for r in trace[last_copy + 1:] if short(r["Kernel_Name"])[0] in APPLY]
    lines = ["# rocprofv3 kernel statistics: bench.py on %s (%s)" % (workload, dtype), "",
             "Command (repository root, MI355X):", "",
             "    rocprofv3 --kernel-trace --stats --output-format csv -d <out>/stats_%s -o run "
             "-- python3 bench.py --workload %s%s --steps 10 --warmup 2 --no-cpu"
             % (workload, workload, dt_flag),
             "", "rocprofv3 statistics (all dispatches of the run, including the conversion-time "
             "timing of kernel shapes and the stream copy):", "",
             "| kernel | calls | avg us | min us | max us | % of GPU time |", "|---|---|---|---|---|---|"]
    for r in stats[:14]:
        lines.append("| %s | %s | %.1f | %.1f | %.1f | %.2f |" % (
            short(r["Name"])[1], r["Calls"], float(r["AverageNs"]) / 1e3,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    # per kernel (full name) over the 12 bench steps after the stream copy
    per = {}
    for r in timed:
        per.setdefault(short(r["Kernel_Name"])[1], []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines += ["", "Applies after the stream copy (the warm-up and timed steps, eager and replayed "
              "from the step's HIP graph), per kernel:", "",
              "| kernel | dispatches | mean us | median us |", "|---|---|---|---|"]
    for k, v in per.items():
        lines.append("| %s | %d | %.1f | %.1f |" % (k, len(v), statistics.mean(v),
                                                    statistics.median(v)))
    js = [l for l in open(os.path.join(out_dir, "stats_%s.log" % workload))
          if l.startswith('{"metric"')]
    if js:
        bench_line = json.loads(js[-1])
        formats = bench_line["config"]["formats"]
        applies = per_format_applies(
            timed, formats, {f: bench_line["formats"][f]["kernels"] for f in formats})
        lines += ["", "One apply per format (the kernels of each format in the warm-up and timed "
                  "steps, summed per apply), beside the bench's own median from HIP "
                  "events in the same run:", "",
                  "| format | kernels | applies | mean us | median us | bench median us |",
                  "|---|---|---|---|---|---|"]
        for f in formats:
            v = applies[f]
            if not v:
                continue
            ts = [t for _, t in v]
            lines.append("| %s | %s | %d | %.1f | %.1f | %.1f |" % (
                f, v[-1][0], len(v), statistics.mean(ts), statistics.median(ts),
                bench_line["formats"][f]["ms_median"] * 1e3))
    open(os.path.join(ROOT, "profiles", "spmv_%s_kernel_stats.md" % tag), "w").write(
        "\n".join(lines) + "\n")
    # ---- traffic per format
    tj = os.path.join(ROOT, "profiles", "traffic.json")
    T = json.load(open(tj)) if os.path.exists(tj) else {}
    T = {k: v for k, v in T.items() if not k.startswith("%s:%s:" % (workload, dtype))}
    fw = ["# HBM traffic per apply: bench.py on %s (%s)" % (workload, dtype), "",
          "Commands (repository root, MI355X; one counter per run, F the format):", "",
          "    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/FETCH_SIZE_%s_F -o run "
          "-- python3 bench.py --workload %s%s --formats F --steps 2 --warmup 1 --no-cpu"
          % (workload, workload, dt_flag),
          "    rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/WRITE_SIZE_%s_F -o run "
          "-- python3 bench.py --workload %s%s --formats F --steps 2 --warmup 1 --no-cpu"
          % (workload, workload, dt_flag),
          "", "(F = csr-K stands for --formats csr --csr-kernel K.)", ""]
    table = ["| format | kernels of one apply | FETCH bytes | WRITE bytes | total |",
             "|---|---|---|---|---|"]
    src_hash = source_hash()
    for f in FORMATS:
        vals = {}
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            d = os.path.join(out_dir, "%s_%s_%s" % (c, workload, f))
            if not os.path.isdir(d):
                break
            rows = sorted(rows_of(d, "counter_collection.csv"), key=lambda r: int(r["Dispatch_Id"]))
            copy = [float(r["Counter_Value"]) * 1024 for r in rows
                    if short(r["Kernel_Name"])[0] == "k_copy"]
            factor = 2.0 * (1 << 30) / statistics.mean(copy)   # copy: 2 GiB read, 2 GiB written
            seq = [(short(r["Kernel_Name"])[0], short(r["Kernel_Name"])[1],
                    float(r["Counter_Value"]) * 1024) for r in rows]
            last = split_apply([(s, full) for s, full, _ in seq])
            tail = seq[-len(last):]
            vals[c] = (factor, [(full, v * factor) for _, full, v in tail])
        if len(vals) < 2:
            continue
        kern = [k for k, _ in vals["FETCH_SIZE"][1]]
        fb = sum(v for _, v in vals["FETCH_SIZE"][1])
        wb = sum(v for _, v in vals["WRITE_SIZE"][1])
        table.append("| %s | %s | %.4g | %.4g | %.4g |" % (f, " + ".join(kern), fb, wb, fb + wb))
        T.setdefault("%s:%s:%s" % (workload, dtype, f.split("-")[0]), []).append({
            "kernels": kern, "bytes_per_launch": round(fb + wb), "fetch_scaled": round(fb),
            "write_scaled": round(wb), "fetch_factor": round(vals["FETCH_SIZE"][0], 5),
            "write_factor": round(vals["WRITE_SIZE"][0], 5), "sources": SOURCES,
            "sha256": src_hash})
    recs = [r for k, v in T.items() if k.startswith("%s:%s:" % (workload, dtype)) for r in v]
    ffs = sorted({r["fetch_factor"] for r in recs}) or [0]
    wfs = sorted({r["write_factor"] for r in recs}) or [0]
    fw.append("Calibration: the library's copy kernel k_copy reads and writes 2 GiB per "
              "dispatch in every run; FETCH_SIZE is scaled by %.4f-%.4f and WRITE_SIZE by "
              "%.4f-%.4f (KiB counters, each run's own factor)." % (ffs[0], ffs[-1], wfs[0], wfs[-1]))
    fw += ["", "Last apply of the timed loop (the run applies only format F):", ""] + table
    open(os.path.join(ROOT, "profiles", "spmv_%s_fetch_write.md" % tag), "w").write(
        "\n".join(fw) + "\n")
    json.dump(T, open(tj, "w"), indent=1, sort_keys=True)
    print("\n".join(fw))


def counters_main():
    """Counter passes of one format: the counters of the last dispatch of each
    kernel of its apply, one table row per kernel."""
    out_dir, workload, fmt = sys.argv[2], sys.argv[3], sys.argv[4]
    dtype = sys.argv[5] if len(sys.argv) > 5 else "f64"
    fmt_base, _, kernel = fmt.partition("-")
    dt_flag = "" if dtype == "f64" else " --dtype " + dtype
    ck_flag = " --csr-kernel " + kernel if kernel else ""
    passes = sorted(d for d in os.listdir(out_dir)
                    if d.startswith("PMC") and d.endswith("_%s_%s" % (workload, fmt))
                    and os.path.isdir(os.path.join(out_dir, d)))
    kern_order, vals, cmds = [], {}, []
    for d in passes:
        names = open(os.path.join(out_dir, d + ".txt")).read().split()
        cmds.append("    rocprofv3 --pmc %s --output-format csv -d <out>/%s -o run -- python3 bench.py "
                    "--workload %s%s --formats %s%s --steps 2 --warmup 1 --no-cpu"
                    % (" ".join(names), d, workload, dt_flag, fmt_base, ck_flag))
        rows = sorted(rows_of(os.path.join(out_dir, d), "counter_collection.csv"),
                      key=lambda r: int(r["Dispatch_Id"]))
        seq, seen_ids = [], set()  # one entry per dispatch (a row per counter)
        for r in rows:
            if r["Dispatch_Id"] not in seen_ids:
                seen_ids.add(r["Dispatch_Id"])
                seq.append((short(r["Kernel_Name"])[0], short(r["Kernel_Name"])[1]))
        dispatch = {}
        for r in rows:  # keep each kernel's last dispatch (the last apply)
            if short(r["Kernel_Name"])[0] in APPLY:
                dispatch[short(r["Kernel_Name"])[1]] = r["Dispatch_Id"]
        last = {full for _, full in split_apply(seq)}
        for r in rows:
            full = short(r["Kernel_Name"])[1]
            if full in last and r["Dispatch_Id"] == dispatch.get(full):
                if full not in kern_order:
                    kern_order.append(full)
                vals.setdefault(full, {})[r["Counter_Name"]] = float(r["Counter_Value"])
    cols = []
    for k in kern_order:
        for c in vals[k]:
            if c not in cols:
                cols.append(c)
    lines = ["# rocprofv3 counters of one apply: bench.py on %s (%s), format %s" % (workload, dtype, fmt),
             "", "Commands (repository root, MI355X; one pass per counter set):", ""] + cmds + [
             "", "The last dispatch of each kernel of the apply (the run applies only this format):", "",
             "| kernel | " + " | ".join(cols) + " |", "|---|" + "---|" * len(cols)]
    for k in kern_order:
        lines.append("| %s | %s |" % (k, " | ".join(
            "%.4g" % vals[k][c] if c in vals[k] else "" for c in cols)))
    path = os.path.join(ROOT, "profiles", "spmv_%s_%s_%s_counters.md" % (workload, dtype, fmt))
    open(path, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "counters":
        counters_main()
    else:
        main()
