"""Decode-step linear-layer benchmark on one MI355X.

One step = one batch-1 decode pass over a model's linear weights: every matrix
y = W . x once, in model order, captured as a HIP graph and replayed.  The
default workload is the TinyLlama-1.1B-shaped weight set (22 layers x {q, k,
v, o, gate, up, down} + output head), run once in bf16 and once in int4-g64;
the value is the achieved HBM rate over the algorithmic bytes of the step.
Inputs are seeded synthetic tensors already resident in HBM.

Prints one JSON line (see the keys below).  --gpus N with N > 1 is refused:
this build measures one GPU.
"""
import argparse
import concurrent.futures
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import memory_bound_weight_amd as L  # noqa: E402
import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, 8 TB/s
METRIC = "achieved HBM GB/s (% of MI355X peak) + equiv. decode tok/s, batch 1"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- byte accounting

def bytes_bf16(N, K, M=1):
    """Algorithmic bytes of one bf16 product: W once, x and y once."""
    return 2 * N * K + 2 * M * K + 4 * M * N


def bytes_q4(N, K, M=1):
    """int4-g64: N*K/2 code bytes + N*K/32 scale bytes, plus x and y."""
    return N * K // 2 + N * K // 32 + 2 * M * K + 4 * M * N


# ---------------------------------------------------------------- weight sets

class Mat:
    def __init__(self, name, layer, idx, N, K):
        self.name, self.layer, self.idx, self.N, self.K = name, layer, idx, N, K


def build_set(model, fmt, dev):
    """Matrices of one decode step, each with its own seeded weights and x."""
    mats = []
    for layer, idx, name, N, K in synth.decode_matrices(model):
        m = Mat(name, layer, idx, N, K)
        W = synth.weight(model["seed"], layer, idx, N, K, device=dev)
        m.x = synth.activation(model["seed"], layer, idx, 1, K, device=dev)
        m.y = torch.empty((1, N), dtype=torch.float32, device=dev)
        if fmt == "bf16":
            m.W = W
            m.bytes = bytes_bf16(N, K)
        else:
            m.Wq, m.S = L.lin_quantize_q4g64(W)
            del W
            m.bytes = bytes_q4(N, K)
        m.fmt = fmt
        mats.append(m)
    torch.cuda.synchronize()
    return mats


def launch(m):
    if m.fmt == "bf16":
        L.lin_gemv_bf16(m.W, m.x, m.y)
    else:
        L.lin_gemv_q4g64(m.Wq, m.S, m.x, m.y)


def kind_of(m):
    return L.LIN_KIND_GEMV_BF16 if m.fmt == "bf16" else L.LIN_KIND_GEMV_Q4G64


def autotune(mats):
    """Load-time tuning: once per distinct (format, N, K), on that shape's first matrix."""
    seen = {}
    for m in mats:
        key = (m.fmt, m.N, m.K)
        if key in seen:
            continue
        if m.fmt == "bf16":
            cfg = L.lin_autotune(L.LIN_KIND_GEMV_BF16, m.W, m.x, m.y)
        else:
            cfg = L.lin_autotune(L.LIN_KIND_GEMV_Q4G64, m.Wq, m.x, m.y, S=m.S)
        seen[key] = cfg
        log("tuned %-5s %6d x %-6d -> %s" % (m.fmt, m.N, m.K, cfg))
    return seen


def capture(mats):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for m in mats:      # one eager pass on the capture stream first
            launch(m)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for m in mats:
            launch(m)
    torch.cuda.synchronize()
    return g


def time_graph(g, steps, warmup):
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    gpu = e0.elapsed_time(e1) / 1000.0 / steps
    return wall, gpu


def variant_key(m):
    c = L.lin_get_config(kind_of(m), 1, m.N, m.K)
    return "%s R%d U%d S%d X%d" % (m.fmt, c["rows"], c["unroll"], c["split"], c["stage_x"])


def kernel_durations(mats, reps=3):
    """Per-launch durations with HIP events on the launch stream (torch's current
    stream, which the binding passes to the library), grouped by kernel variant."""
    per = {}
    stream = torch.cuda.current_stream()
    for _ in range(reps):
        evs = []
        for m in mats:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            launch(m)
            b.record(stream)
            evs.append((m, a, b))
        torch.cuda.synchronize()
        for m, a, b in evs:
            d = per.setdefault(variant_key(m), {"t": 0.0, "bytes": 0, "n": 0, "shapes": set()})
            d["t"] += a.elapsed_time(b) / 1000.0
            d["bytes"] += m.bytes
            d["n"] += 1
            d["shapes"].add("%dx%d" % (m.N, m.K))
    return per


# ---------------------------------------------------------------- CPU baseline

def cpu_baseline(model, layers, threads):
    """The oracle, as it stands, on the host cores: a bounded sample (the first
    `layers` layers, bf16 and int4-g64), rows split over `threads` threads."""
    import oracle
    work = []
    for layer, idx, name, N, K in synth.decode_matrices(model):
        if layer >= layers:
            continue
        W = synth.bits(synth.weight(model["seed"], layer, idx, N, K))
        x = synth.bits(synth.activation(model["seed"], layer, idx, 1, K))
        Wq, S = oracle.quantize_q4g64(W)
        work.append(("bf16", W, None, x, bytes_bf16(N, K)))
        work.append(("q4", Wq, S, x, bytes_q4(N, K)))
    total_bytes = sum(w[4] for w in work)

    def run_rows(item, lo, hi):
        fmt, A, S, x, _ = item
        if fmt == "bf16":
            oracle.gemm_dense(A[lo:hi], x)
        else:
            oracle.gemm_q4g64(A[lo:hi], S[lo:hi], x)

    jobs = []
    for item in work:
        N = item[1].shape[0]
        step = max(1, N // (4 * threads))
        jobs += [(item, lo, min(N, lo + step)) for lo in range(0, N, step)]
    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda j: run_rows(*j), jobs))
    dt = time.perf_counter() - t0
    return {"value": round(total_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": "%s layers 0-%d (%d matrices), bf16 and int4-g64, %.1f MB of weights, "
                      "batch 1, fp64 sequential sums, %.2f s wall"
                      % (model["name"], layers - 1, len(work) // 2, total_bytes / 1e6, dt)}


# ---------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="tinyllama", choices=["tinyllama", "qwen7b"])
    ap.add_argument("--no-tune", action="store_true")
    ap.add_argument("--cpu-layers", type=int, default=4)
    ap.add_argument("--skip-cpu", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the decode-step linear layer is built and timed on a "
              "single MI355X; --gpus %d is not supported." % args.gpus, file=sys.stderr)
        sys.exit(2)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    model = synth.TINYLLAMA if args.workload == "tinyllama" else synth.QWEN7B
    log("building %s weight sets on %s" % (model["name"], torch.cuda.get_device_name(dev)))
    sets = {f: build_set(model, f, dev) for f in ("bf16", "q4")}
    allm = sets["bf16"] + sets["q4"]
    tuned = {} if args.no_tune else autotune(allm)

    graphs = {f: capture(sets[f]) for f in sets}
    g_all = capture(allm)
    per_fmt = {}
    for f in ("bf16", "q4"):
        wall, gpu = time_graph(graphs[f], max(5, args.steps // 2), args.warmup)
        b = sum(m.bytes for m in sets[f])
        per_fmt[f] = {"ms_per_token": round(gpu * 1e3, 4), "equiv_tok_s": round(1.0 / gpu, 1),
                      "GB_s": round(b / gpu / 1e9, 1), "bytes": b}
        log("%s step: %.1f us, %.1f GB/s, %.0f tok/s" % (f, gpu * 1e6, b / gpu / 1e9, 1 / gpu))

    # the timed region: K steps of the whole path (bf16 + int4 sets)
    torch.cuda.synchronize()
    wall, gpu = time_graph(g_all, args.steps, args.warmup)
    step_bytes = sum(m.bytes for m in allm)
    gbs = step_bytes / wall / 1e9

    per = kernel_durations(allm)
    dom_key = max(per, key=lambda k: per[k]["t"])
    dom = per[dom_key]
    achieved = dom["bytes"] / dom["t"] / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": dom_key, "launches": dom["n"], "shapes": sorted(dom["shapes"]),
                "avg_launch_us": round(dom["t"] / dom["n"] * 1e6, 3),
                "bytes_per_launch": int(dom["bytes"] / dom["n"])}

    out = {"metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16 and int4-g64 weights, bf16 x, fp32 accumulate", "data": "synthetic",
           "config": {"workload": "%s decode weight set, batch 1, bf16 + int4-g64 (%d matrices each)"
                      % (model["name"], len(sets["bf16"])), "batch": 1,
                      "matrices_per_step": len(allm), "bytes_per_step": step_bytes,
                      "tuned": not args.no_tune},
           "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
           "gpu_ms_per_step": round(gpu * 1e3, 4),
           "per_format": per_fmt, "roofline": roofline}
    if not args.skip_cpu:
        out["cpu_baseline"] = cpu_baseline(model, args.cpu_layers, min(16, os.cpu_count() or 1))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
