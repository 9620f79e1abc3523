"""Build hbm_traffic.json (HBM bytes per GEMV dispatch) from rocprofv3 counter runs.

The table is what bench.py reports as a kernel's measured HBM traffic beside its
algorithmic bytes.  Inputs, all written by rocprofv3 with --output-format csv:

  --fetch / --write        FETCH_SIZE and WRITE_SIZE runs (one counter per run) of
                           `python -u bench.py --counter-pass [--workload ... --formats ...]`
  --copy-fetch / --copy-write
                           the same counters over `python -u bench.py --copy-calibration BYTES`
  --launches               the log of one of the counter-pass runs (its JSON line
                           lists every launch of a pass, in order: variant, shape)

Both counters read KiB per dispatch.  Each is scaled so that a plain device copy
of BYTES reads (FETCH_SIZE) and writes (WRITE_SIZE) exactly BYTES; the scale is
stored with the entry.  The counter pass launches the step twice; the last pass's
GEMV dispatches are matched to the launch list in order, and the median over the
launches of one (variant, shape) is kept.  An entry holds the hash of the sources
its kernels are built from: bench.py ignores it once those change.

Example (repository root):

  python memory_bound_weight_amd/tuning/hbm_counters.py --fetch prof/pa_fetch \\
      --write prof/pa_write --copy-fetch prof/pa_cfetch \\
      --copy-write prof/pa_cwrite --copy-bytes 1073741824 \\
      --launches prof/counter_pass.log --out memory_bound_weight_amd/tuning/hbm_traffic.json
"""
import argparse
import collections
import csv
import hashlib
import json
import os
import re
import statistics

PKG = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COMMON = ["csrc/kern_common.h"]


def sources(variant):
    """Source files the kernel of a GEMV variant string is compiled from."""
    fam, *fields = variant.split()
    x = int(re.search(r"X(\d+)", variant).group(1))
    if fam == "gemv_bf16":
        return ["csrc/gemv_bf16.hip", "csrc/gemv_bf16_impl.h"] + COMMON
    if fam == "gemv_i8":
        return ["csrc/gemv_i8.hip", "csrc/gemv_i8_impl.h"] + COMMON
    if fam == "gemv_q4g64" and x == 2:
        return ["csrc/gemv_q4x.hip"] + COMMON
    if fam == "gemv_q4g64":
        return ["csrc/gemv_q4g64.hip", "csrc/gemv_q4g64_impl.h"] + COMMON
    raise ValueError("no source list for variant %r" % variant)


def expected_instance(variant):
    """Pattern of the kernel instance a GEMV variant string launches (no epilogue,
    no prologue): the function and the template arguments the variant fixes."""
    fam = variant.split()[0]
    R, U, S, X = (int(re.search(f + r"(\d+)", variant).group(1)) for f in ("R", "U", "S", "X"))
    if fam == "gemv_q4g64" and X == 2:
        return r"gemv_q4_xres<\d+, %d, %d, %d, 0>" % (S, U, R)
    fn = {"gemv_bf16": "gemv_bf16_valu", "gemv_i8": "gemv_i8_valu", "gemv_q4g64": "gemv_q4_valu"}[fam]
    return r"%s<1, %d, %d, %d, %s, 0, false>" % (fn, R, U, S, "true" if X else "false")


def source_hash(paths):
    src = b"".join(open(os.path.join(PKG, p), "rb").read() for p in paths)
    return hashlib.sha256(src).hexdigest()[:16]


def dispatches(run_dir, counter):
    """[(dispatch id, kernel name, value)] of one counter, in dispatch order."""
    path = os.path.join(run_dir, "pmc_counter_collection.csv")
    acc = collections.OrderedDict()
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        name, v = acc.get(d, (r["Kernel_Name"], 0.0))
        acc[d] = (name, v + float(r["Counter_Value"]))
    return [(d, n, v) for d, (n, v) in sorted(acc.items())]


def copy_scale(run_dir, counter, nbytes):
    vals = [v for _, n, v in dispatches(run_dir, counter) if "copyBuffer" in n or "copy" in n.lower()]
    if not vals:
        raise SystemExit("no copy dispatch in %s" % run_dir)
    return nbytes / (statistics.median(vals) * 1024.0)


def short(name):
    name = name.replace("void ", "").replace("(lin::KArgs)", "")
    return name.replace("lin::(anonymous namespace)::", "").replace("lin::", "")


def last_pass(run_dir, counter, seq):
    """The last len(seq) GEMV dispatches of a counter-pass run, paired with seq."""
    g = [(d, n, v) for d, n, v in dispatches(run_dir, counter) if "gemv" in n]
    if len(g) < 2 * len(seq):
        raise SystemExit("%s: %d GEMV dispatches, expected two passes of %d"
                         % (run_dir, len(g), len(seq)))
    return list(zip(seq, g[-len(seq):]))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    for a in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--launches", "--out"):
        ap.add_argument(a, required=True)
    ap.add_argument("--copy-bytes", type=int, required=True)
    args = ap.parse_args()
    seq = None
    for line in open(args.launches):
        if line.startswith("{") and "counter_pass" in line:
            seq = [tuple(x) for x in json.loads(line)["counter_pass"]]
    if not seq:
        raise SystemExit("no counter-pass launch list in %s" % args.launches)
    fs = copy_scale(args.copy_fetch, "FETCH_SIZE", args.copy_bytes)
    ws = copy_scale(args.copy_write, "WRITE_SIZE", args.copy_bytes)
    per = collections.defaultdict(lambda: collections.defaultdict(lambda: {"f": [], "w": []}))
    names = collections.defaultdict(set)
    for counter, run, slot, scale in (("FETCH_SIZE", args.fetch, "f", fs),
                                      ("WRITE_SIZE", args.write, "w", ws)):
        for key, (d, name, v) in last_pass(run, counter, seq):
            if not re.search(expected_instance(key[0]), short(name)):
                raise SystemExit("%s dispatch %d is %s, but the launch list has %s there: the "
                                 "launch list and the dispatches do not line up"
                                 % (counter, d, short(name), key[0]))
            per[key[0]][key[1]][slot].append(v * 1024.0 * scale)
            names[key[0]].add(short(name).split("<")[0])

    old = []
    if os.path.exists(args.out):
        with open(args.out) as f:
            old = json.load(f)["measured"]
    # entries whose kernel sources changed since they were measured are dropped
    table = {e["kernel"]: e for e in old
             if e.get("sources") and e["src_sha256_16"] == source_hash(e["sources"])}
    for variant, shapes in per.items():
        if len(names[variant]) != 1:
            raise SystemExit("variant %s matched kernels %s: the launch list and the dispatches "
                             "do not line up" % (variant, sorted(names[variant])))
        srcs = sources(variant)
        e = table.get(variant)
        if e is None or e["src_sha256_16"] != source_hash(srcs):
            e = {"kernel": variant, "per_shape": {}}
        e.update({"function": names[variant].pop(), "src_sha256_16": source_hash(srcs),
                  "fetch_scale": round(fs, 4), "write_scale": round(ws, 4), "sources": srcs})
        for shape, d in shapes.items():
            e["per_shape"][shape] = {"fetch_bytes": int(statistics.median(d["f"])),
                                     "write_bytes": int(statistics.median(d["w"])),
                                     "dispatches": len(d["f"])}
        table[variant] = e
    out = {"measured": sorted(table.values(), key=lambda e: e["kernel"]),
           "note": "HBM bytes per dispatch from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE on MI355X "
                   "over bench.py --counter-pass, scaled by what the same counters read for a "
                   "plain device copy of known size; valid only while the kernel sources hash "
                   "to src_sha256_16"}
    with open(args.out, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    for e in out["measured"]:
        for shape, d in sorted(e["per_shape"].items()):
            print("%-26s %-12s fetch %12d  write %10d  (%d dispatches)"
                  % (e["kernel"], shape, d["fetch_bytes"], d["write_bytes"], d.get("dispatches", 0)))


if __name__ == "__main__":
    main()
