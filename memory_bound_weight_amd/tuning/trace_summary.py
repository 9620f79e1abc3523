"""Summarise a rocprofv3 kernel trace of a bench.py decode-step run as markdown.

Inputs, written by `rocprofv3 --kernel-trace --stats -d DIR -o NAME --output-format csv
-- python -u bench.py ...`:

  --trace DIR/NAME   prefix of NAME_kernel_stats.csv and NAME_kernel_trace.csv
  --bench LOG        the stdout of a bench.py run of the same workload (its JSON
                     line lists every kernel variant of the step with its shape and
                     the duration bench.py measured live with HIP events)

Output: the profiler's top kernels (from the stats file), then one row per kernel
variant and shape of the step: the average and median duration of the traced
dispatches of that kernel instance at that shape's grid, beside bench.py's own
figure.  The grid (work-items) of a shape follows from the variant's launch
geometry, restated here for the GEMV families the decode step uses.  With
--reduced OUT the per-(kernel, grid) dispatch statistics are also written as a
small CSV, so that the raw trace need not be kept.

Example (repository root):

  python memory_bound_weight_amd/tuning/trace_summary.py --trace prof/pa_qwen/bench \\
      --bench prof/bench.log --out prof/kernel_stats.md
"""
import argparse
import collections
import csv
import json
import re
import statistics

BLOCK = 256   # threads per workgroup of the GEMV kernels
CUS = 256     # compute units of an MI355X (the int4 x-resident grid is a multiple of them)


def instance_pattern(variant):
    """Regex of the kernel instance a GEMV variant string launches (no epilogue,
    no prologue)."""
    fam = variant.split()[0]
    R, U, S, X = (int(re.search(f + r"(\d+)", variant).group(1)) for f in ("R", "U", "S", "X"))
    if fam == "gemv_q4g64" and X == 2:
        return r"gemv_q4_xres<\d+, %d, %d, %d, 0>" % (S, U, R)
    fn = {"gemv_bf16": "gemv_bf16_valu", "gemv_i8": "gemv_i8_valu", "gemv_q4g64": "gemv_q4_valu"}[fam]
    return r"%s<1, %d, %d, %d, %s, 0, false>" % (fn, R, U, S, "true" if X else "false")


def grid_items(variant, N):
    """Work-items of one launch of a GEMV variant on N rows at batch 1: a
    workgroup holds 4/S row groups of R rows; the x-resident int4 family rounds
    its workgroup count up to whole compute units."""
    fam = variant.split()[0]
    R, S, X = (int(re.search(f + r"(\d+)", variant).group(1)) for f in ("R", "S", "X"))
    per = R * (4 // S)
    blocks = -(-N // per)
    if fam == "gemv_q4g64" and X == 2:
        blocks = -(-blocks // CUS) * CUS
    return blocks * BLOCK


def short(name):
    name = name.replace("void ", "").replace("(lin::KArgs)", "")
    return name.replace("lin::(anonymous namespace)::", "").replace("lin::", "")


def col(row, *names):
    for n in names:
        if n in row and row[n] != "":
            return row[n]
    raise KeyError(names[0])


def grid_of(row):
    """Work-items of a traced dispatch (the product of the grid's dimensions;
    a missing or empty Y or Z column counts as 1)."""
    g = int(col(row, "Grid_Size_X", "Grid_Size"))
    for d in ("Grid_Size_Y", "Grid_Size_Z"):
        if row.get(d, "") != "":
            g *= int(row[d])
    return g


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--trace", required=True)
    ap.add_argument("--bench", required=True)
    ap.add_argument("--out", required=True)
    ap.add_argument("--reduced", default=None)
    ap.add_argument("--from-reduced", default=None, metavar="CSV",
                    help="take the per-(kernel, grid) dispatch statistics from a CSV that an "
                         "earlier run wrote with --reduced instead of NAME_kernel_trace.csv")
    ap.add_argument("--top", type=int, default=12)
    args = ap.parse_args()

    bench = None
    for line in open(args.bench):
        if line.startswith("{") and '"kernels"' in line:
            bench = json.loads(line)
    if bench is None:
        raise SystemExit("no bench.py JSON line with per-kernel figures in %s" % args.bench)

    stats = list(csv.DictReader(open(args.trace + "_kernel_stats.csv")))
    # (kernel, grid) -> (dispatches, mean us, median us, min us, max us)
    groups = {}
    if args.from_reduced:
        for r in csv.DictReader(open(args.from_reduced)):
            groups[(r["kernel"], int(r["grid_items"]))] = (
                int(r["dispatches"]), float(r["avg_us"]), float(r["median_us"]),
                float(r["min_us"]), float(r["max_us"]))
    else:
        durs = collections.defaultdict(list)
        for r in csv.DictReader(open(args.trace + "_kernel_trace.csv")):
            name = short(col(r, "Kernel_Name"))
            d = (int(col(r, "End_Timestamp")) - int(col(r, "Start_Timestamp"))) / 1000.0
            durs[(name, grid_of(r))].append(d)
        for key, v in durs.items():
            groups[key] = (len(v), statistics.mean(v), statistics.median(v), min(v), max(v))

    out = []
    out.append("Top kernels from `%s_kernel_stats.csv` (every dispatch of the run):\n" % args.trace.split("/")[-1])
    out.append("| kernel | calls | avg us | min us | max us | % of GPU time |")
    out.append("|---|---|---|---|---|---|")
    stats.sort(key=lambda r: -float(r["TotalDurationNs"]))
    for r in stats[:args.top]:
        nm = short(r["Name"])
        nm = nm if len(nm) <= 70 else nm[:67] + "..."
        out.append("| `%s` | %s | %.2f | %.2f | %.2f | %.2f |" % (
            nm, r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    out.append("")
    out.append("Per kernel of the step: the traced dispatches of its instance at its shape's grid, "
               "beside bench.py's live figure (HIP events around graph replays holding only that "
               "kernel's launches).\n")
    out.append("| kernel variant | shape | instance | launches per step | rocprof dispatches | "
               "rocprof avg us | rocprof median us | bench.py live us | difference |")
    out.append("|---|---|---|---|---|---|---|---|---|")
    # shapes of one variant with the same N launch the same instance on the same
    # grid: their dispatches cannot be told apart, and the row says so
    same = collections.defaultdict(list)
    for key in bench["kernels"]:
        variant, shape = key.rsplit(" ", 1)
        same[(variant, grid_items(variant, int(shape.split("x")[0])))].append(shape)
    for key, k in bench["kernels"].items():
        variant, shape = key.rsplit(" ", 1)
        N = int(shape.split("x")[0])
        pat = re.compile(instance_pattern(variant))
        g = grid_items(variant, N)
        others = [o for o in same[(variant, g)] if o != shape]
        hits = [(n, v) for (n, gr), v in groups.items() if gr == g and pat.search(n)]
        if len(hits) != 1:
            out.append("| `%s` | %s | (%d matching instances at grid %d) | %d | | | | %.2f | |"
                       % (variant, shape, len(hits), g, k["launches"], k["avg_us"]))
            continue
        n, (cnt, avg, med, _, _) = hits[0]
        diff = "%.1f %%" % (100.0 * (avg - k["avg_us"]) / k["avg_us"])
        if others:
            diff = "(traced with %s: same instance and grid)" % ", ".join(others)
        out.append("| `%s` | %s | `%s` | %d | %d | %.2f | %.2f | %.2f | %s |" % (
            variant, shape, n, k["launches"], cnt, avg, med, k["avg_us"], diff))
    with open(args.out, "w") as f:
        f.write("\n".join(out) + "\n")
    if args.reduced:
        with open(args.reduced, "w", newline="") as f:
            w = csv.writer(f)
            w.writerow(["kernel", "grid_items", "dispatches", "avg_us", "median_us", "min_us", "max_us"])
            for (n, gr), (cnt, avg, med, lo, hi) in sorted(groups.items(),
                                                          key=lambda kv: -kv[1][0] * kv[1][1]):
                w.writerow([n, gr, cnt, round(avg, 3), round(med, 3), round(lo, 3), round(hi, 3)])
    print("\n".join(out))


if __name__ == "__main__":
    main()
