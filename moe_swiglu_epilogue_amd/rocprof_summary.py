"""Turn rocprofv3 CSV output into the short text/JSON summaries kept under
profiles/.

  stats: kernel-trace statistics (calls, average/min/max duration per kernel)
         from a `rocprofv3 --kernel-trace --stats -f csv` run.
  counters: the per-dispatch average of every counter in a `--pmc` run, for
         one kernel.
  pmc:   HBM traffic of one kernel from two counter runs
         (`--pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`, both in KiB per
         dispatch), each scaled by what the same counter reads for the
         calibration copy kernel, which moves a known number of bytes.

Usage:
  python -m moe_swiglu_epilogue_amd.rocprof_summary stats DIR OUT.txt --cmd "..."
  python -m moe_swiglu_epilogue_amd.rocprof_summary counters DIR [DIR ...] --out OUT.txt \\
      --kernel K --cmd "..."
  python -m moe_swiglu_epilogue_amd.rocprof_summary pmc FETCH_DIR WRITE_DIR OUT \\
      --kernel K --calib calib_copy_kernel --calib-bytes-each-way N \\
      --alg-bytes N --source-sha256 H --cmd "..."
"""
import argparse
import csv
import glob
import json
import os
import statistics
import sys


def _one(dir_, suffix):
    hits = sorted(glob.glob(os.path.join(dir_, "**", "*" + suffix), recursive=True))
    if not hits:
        raise SystemExit("no *%s under %s" % (suffix, dir_))
    return hits


def _short(name):
    """'void (anonymous namespace)::k<(anonymous namespace)::A, true>(args)' ->
    'k<A, true>'."""
    n = name.replace("(anonymous namespace)::", "")
    depth, cut = 0, len(n)
    for i, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    n = n[:cut].strip()
    return n[5:] if n.startswith("void ") else n


def stats(args):
    rows = []
    for path in _one(args.dir, "kernel_stats.csv"):
        with open(path) as f:
            rows += list(csv.DictReader(f))
    lines = ["# rocprofv3 kernel-trace statistics", "", "command:", "  " + args.cmd, "",
             "%-40s %6s %12s %12s %12s %7s" % ("kernel", "calls", "avg_us", "min_us", "max_us", "pct")]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append("%-40s %6s %12.3f %12.3f %12.3f %7.2f" % (
            _short(r["Name"])[:40], r["Calls"], float(r["AverageNs"]) / 1e3,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    if args.clusters:
        lines += ["", "duration clusters of %s (calls sorted by duration, split where one is"
                  " more than %.1fx the one before)" % (args.clusters, args.gap),
                  "%-12s %6s %12s %12s %12s %12s" % ("cluster", "calls", "avg_us", "p50_us",
                                                     "min_us", "max_us")]
        for k, c in enumerate(_clusters(args.dir, args.clusters, args.gap)):
            lines.append("%-12d %6d %12.3f %12.3f %12.3f %12.3f" % (
                k, len(c), statistics.fmean(c), statistics.median(c), c[0], c[-1]))
    text = "\n".join(lines) + "\n"
    with open(args.out, "w") as f:
        f.write(text)
    print(text)


def _clusters(dir_, kernel, gap):
    """Durations (us) of one kernel's dispatches from the kernel trace, sorted
    and split into groups wherever a duration exceeds the previous one by
    more than the factor `gap` (one kernel launched on inputs of very
    different sizes, with the same grid)."""
    d = []
    for path in _one(dir_, "kernel_trace.csv"):
        with open(path) as f:
            for r in csv.DictReader(f):
                if _short(r["Kernel_Name"]) == kernel:
                    d.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    d.sort()
    out, cur = [], []
    for v in d:
        if cur and v > gap * cur[-1]:
            out.append(cur)
            cur = []
        cur.append(v)
    if cur:
        out.append(cur)
    return out


def _counter(dir_, counter):
    per = {}
    for path in _one(dir_, "counter_collection.csv"):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") != counter:
                    continue
                per.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return per


def pmc(args):
    fetch = _counter(args.fetch_dir, "FETCH_SIZE")
    write = _counter(args.write_dir, "WRITE_SIZE")

    def avg(d, k):
        hit = [v for name, vs in d.items() if name.startswith(k) for v in vs]
        if not hit:
            raise SystemExit("kernel %s not found (have %s)" % (k, sorted(d)))
        return statistics.mean(hit), len(hit)

    kf, nkf = avg(fetch, args.kernel)
    kw, nkw = avg(write, args.kernel)
    cf, _ = avg(fetch, args.calib)
    cw, _ = avg(write, args.calib)
    f_scale = args.calib_bytes_each_way / (cf * 1024.0)
    w_scale = args.calib_bytes_each_way / (cw * 1024.0)
    fetch_b = kf * 1024.0 * f_scale
    write_b = kw * 1024.0 * w_scale
    out = {
        "kernel": args.kernel,
        "kernel_source_sha256": args.source_sha256,
        "dispatches": {"fetch": nkf, "write": nkw},
        "fetch_kib_per_dispatch": round(kf, 1),
        "write_kib_per_dispatch": round(kw, 1),
        "calib_kernel": args.calib,
        "calib_bytes_read_and_written_each": args.calib_bytes_each_way,
        "calib_fetch_kib": round(cf, 1), "calib_write_kib": round(cw, 1),
        "fetch_scale": round(f_scale, 5), "write_scale": round(w_scale, 5),
        "traffic_bytes_per_launch": int(round(fetch_b + write_b)),
        "traffic_read_bytes": int(round(fetch_b)), "traffic_write_bytes": int(round(write_b)),
        "alg_bytes_per_launch": args.alg_bytes,
        "traffic_over_alg": round((fetch_b + write_b) / args.alg_bytes, 4),
        "command": args.cmd,
    }
    with open(args.out + ".json", "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    text = ["# rocprofv3 HBM counters: %s" % args.kernel, "", "commands:", "  " + args.cmd, ""]
    text += ["%-28s %s" % (k, v) for k, v in out.items() if k != "command"]
    with open(args.out + ".txt", "w") as f:
        f.write("\n".join(text) + "\n")
    print("\n".join(text))


def counters(args):
    per = {}
    for d in args.dirs:
        for path in _one(d, "counter_collection.csv"):
            with open(path) as f:
                for r in csv.DictReader(f):
                    if _short(r["Kernel_Name"]).startswith(args.kernel):
                        per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if not per:
        raise SystemExit("kernel %s not found" % args.kernel)
    lines = ["# rocprofv3 counters: %s (average per dispatch)" % args.kernel, "", "commands:",
             "  " + args.cmd, "", "%-28s %10s %18s" % ("counter", "dispatches", "average")]
    for name in sorted(per):
        lines.append("%-28s %10d %18.2f" % (name, len(per[name]), statistics.mean(per[name])))
    text = "\n".join(lines) + "\n"
    with open(args.out, "w") as f:
        f.write(text)
    print(text)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    a = sub.add_parser("stats")
    a.add_argument("dir")
    a.add_argument("out")
    a.add_argument("--cmd", required=True)
    a.add_argument("--clusters", metavar="KERNEL",
                   help="also split this kernel's dispatches into duration clusters")
    a.add_argument("--gap", type=float, default=1.5)
    b = sub.add_parser("pmc")
    b.add_argument("fetch_dir")
    b.add_argument("write_dir")
    b.add_argument("out", help="output path without extension (.json and .txt are written)")
    b.add_argument("--kernel", required=True)
    b.add_argument("--calib", required=True)
    b.add_argument("--calib-bytes-each-way", type=int, required=True,
                   help="bytes the copy kernel reads per dispatch (it writes as many)")
    b.add_argument("--alg-bytes", type=int, required=True)
    b.add_argument("--source-sha256", required=True)
    b.add_argument("--cmd", required=True)
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--out", required=True)
    c.add_argument("--kernel", required=True)
    c.add_argument("--cmd", required=True)
    args = ap.parse_args(argv)
    {"stats": stats, "pmc": pmc, "counters": counters}[args.what](args)


if __name__ == "__main__":
    main(sys.argv[1:])
