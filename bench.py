"""Decode-step linear-layer benchmark on one MI355X.

One step = one batch-1 decode pass over a model's linear weights: every matrix
y = W . x once, in model order (q|k|v and gate|up concatenated at load), each
format's pass captured as a HIP graph and replayed (the timed step: one graph
of all formats' passes).  The
default workload is the Qwen2.5-7B-shaped weight set (28 layers x {q, k, v,
o, gate, up, down} + output head, 14.1 GB in bf16), run once in bf16 and once
in int4-g64; the value is the achieved HBM rate over the algorithmic bytes of
the step.  --workload tinyllama runs the TinyLlama-1.1B-shaped set.
Inputs are seeded synthetic tensors already resident in HBM.

Prints one JSON line (see the keys below).  --gpus N with N > 1 is refused:
the benchmark measures one GPU.
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
# worker threads of the oracle's timed sample: the host's share for one GPU
CPU_THREADS = min(16, os.cpu_count() or 1)
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


def bytes_i8(N, K, M=1):
    """INT8: N*K code bytes + 4*N scale bytes (one fp32 per row), plus x and y."""
    return N * K + 4 * N + 2 * M * K + 4 * M * N


# ---------------------------------------------------------------- weight sets

class Mat:
    """One launch: a matrix (or load-time concatenation of matrices sharing x)."""

    def __init__(self, name, layer, N, K):
        self.name, self.layer, self.N, self.K = name, layer, N, K


def build_set(model, fmt, dev, fused=True):
    """Matrices of one decode step, each part with its own seeded weights; one
    seeded x per launch group."""
    mats = []
    for layer, parts in synth.decode_groups(model, fused):
        K = parts[0][3]
        N = sum(p[2] for p in parts)
        m = Mat("|".join(p[1] for p in parts), layer, N, K)
        W = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
        r = 0
        for idx, name, n, k in parts:
            W[r:r + n] = synth.weight(model["seed"], layer, idx, n, k, device=dev)
            r += n
        m.x = synth.activation(model["seed"], layer, parts[0][0], 1, K, device=dev)
        m.y = torch.empty((1, N), dtype=torch.float32, device=dev)
        if fmt == "bf16":
            m.W = W
            m.bytes = bytes_bf16(N, K)
        elif fmt == "q4":
            m.Wq, m.S = L.lin_quantize_q4g64(W)
            del W
            m.bytes = bytes_q4(N, K)
        else:
            m.Wq, m.S = L.lin_quantize_i8(W)
            del W
            m.bytes = bytes_i8(N, K)
        m.fmt = fmt
        mats.append(m)
    torch.cuda.synchronize()
    return mats


def launch(m):
    if m.fmt == "bf16":
        L.lin_gemv_bf16(m.W, m.x, m.y)
    elif m.fmt == "q4":
        L.lin_gemv_q4g64(m.Wq, m.S, m.x, m.y)
    else:
        L.lin_gemv_i8(m.Wq, m.S, m.x, m.y)


KINDS = {"bf16": L.LIN_KIND_GEMV_BF16, "q4": L.LIN_KIND_GEMV_Q4G64, "i8": L.LIN_KIND_GEMV_I8}
KERNEL_NAMES = {"bf16": "gemv_bf16", "q4": "gemv_q4g64", "i8": "gemv_i8"}
FORMAT_NAMES = {"bf16": "bf16", "q4": "int4-g64", "i8": "INT8 (fp32 scale per row)"}


def kind_of(m):
    return KINDS[m.fmt]


def tune_key(m):
    return (kind_of(m), 1, m.N, m.K)


NORM_KINDS = {"bf16": L.LIN_KIND_GEMV_BF16_NORM, "q4": L.LIN_KIND_GEMV_Q4G64_NORM,
              "i8": L.LIN_KIND_GEMV_I8_NORM}
NORM_OF = ("q|k|v", "gate|up", "head")   # projections whose input is RMS-normalised


def tune_keys(m, norms=False):
    """Tuning keys a matrix is launched under: its product and, with norms, the
    RMSNorm-prologue product of the normalised projections."""
    keys = [tune_key(m)]
    if norms and m.name in NORM_OF and m.fmt in NORM_KINDS:
        keys.append((NORM_KINDS[m.fmt], 1, m.N, m.K))
    return keys


def autotune(mats, only=None, norms=False):
    """Load-time tuning: once per distinct (kind, N, K), with lin_autotune_set
    over all of that shape's matrices (the layers), timed back to back the way
    the step runs them; returns {tune key: config}."""
    groups = {}
    for m in mats:
        for key in tune_keys(m, norms):
            if only is None or key in only:
                groups.setdefault(key, []).append(m)
    seen = {}
    for key, ms in groups.items():
        # time every candidate over more distinct weights than the caches hold,
        # as the step streams them (a shape's layers alone may fit the 256 MB
        # Infinity Cache)
        ms = with_copies(ms, 600 << 20)
        m = ms[0]
        if m.fmt == "bf16":
            cfg = L.lin_autotune_set(key[0], [g.W for g in ms], m.x, m.y)
        else:
            cfg = L.lin_autotune_set(key[0], [g.Wq for g in ms], m.x, m.y, Ss=[g.S for g in ms])
        seen[key] = cfg
        log("tuned kind %d %-5s %6d x %-6d over %d matrices -> %s" % (key[0], m.fmt, m.N, m.K,
                                                                    len(ms), cfg))
        del ms
    return seen


def apply_tuning(mats, path, retune, norms=False, save_to=None):
    """Use the persisted tuning table (tuned once with lin_autotune on MI355X);
    keys it does not cover, or all keys with retune, are tuned now.  save_to:
    also write the table with the keys tuned now."""
    keys = {k for m in mats for k in tune_keys(m, norms)}
    if retune or not os.path.exists(path):
        entries = autotune(mats, norms=norms)
        L.save_tuning(save_to or path, entries)
        return "tuned now (%d shapes), saved to %s" % (len(entries),
                                                       os.path.relpath(save_to or path, ROOT))
    ok, stale = L.load_tuning(path)
    missing = keys - set(ok)
    if missing:
        new = autotune(mats, only=missing, norms=norms)
        if save_to:
            with open(path) as f:
                old = {(e["kind"], e["M"], e["N"], e["K"]): e["cfg"] for e in json.load(f)["entries"]}
            old.update(new)
            L.save_tuning(save_to, old)
    return "loaded %s (%d shapes%s)" % (os.path.relpath(path, ROOT), len(keys - missing),
                                        ", %d tuned now" % len(missing) if missing else "")


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


def time_runs(fns, steps, warmup):
    """Wall and GPU (event) time per step of calling every fn in order."""
    for _ in range(warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        for f in fns:
            f()
    e1.record()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps, e0.elapsed_time(e1) / 1000.0 / steps


def time_graph(g, steps, warmup):
    warm(g)
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
    return "%s R%d U%d S%d X%d" % (KERNEL_NAMES[m.fmt], c["rows"], c["unroll"], c["split"],
                                   c["stage_x"])


WARM_S = 0.25   # steady state: replay a fresh graph this long before timing it


def warm(g, seconds=WARM_S):
    """Replay a graph for about `seconds`.  The first passes over freshly
    allocated weights run slower (measured: the Qwen2.5-7B bf16 pass 2.31 ms for
    its first ~0.1 s, 2.20 ms from then on, also after an idle pause), so every
    timed graph is first brought to that steady state."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            g.replay()
        torch.cuda.synchronize()


def replay_times(g, reps, warmup):
    """Durations (s) of `reps` replays of a graph, each bracketed by its own HIP
    events on the stream the replays run on, after `warmup` replays and the
    steady-state warm-up above."""
    warm(g)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) / 1000.0 for a, b in ev]


def counter_pass(mats):
    """Two eager passes over the step's launches, in step order, one dispatch per
    launch, for a profiler's per-dispatch counters; prints the launch list
    (variant, shape) that the counter converter matches the last pass against."""
    seq = [[variant_key(m), "%dx%d" % (m.N, m.K)] for m in mats]
    for _ in range(2):
        for m in mats:
            launch(m)
        torch.cuda.synchronize()
    print(json.dumps({"counter_pass": seq, "passes": 2}), flush=True)


def quartiles(ts):
    q1, q2, q3 = np.percentile(np.asarray(ts, dtype=np.float64), [25, 50, 75])
    return q2, q3 - q1


def with_copies(ms, min_bytes):
    """The matrices ms, plus clones of their weights (sharing x and y) until the
    list holds at least min_bytes of distinct weights, so that back-to-back
    launches over it stream from HBM rather than the 256 MB Infinity Cache."""
    out = list(ms)
    i = 0
    while sum(m.bytes for m in out) < min_bytes:
        src = ms[i % len(ms)]
        c = Mat(src.name, src.layer, src.N, src.K)
        c.x, c.y, c.fmt, c.bytes = src.x, src.y, src.fmt, src.bytes
        if src.fmt == "bf16":
            c.W = src.W.clone()
        else:
            c.Wq, c.S = src.Wq.clone(), src.S.clone()
        out.append(c)
        i += 1
    return out


def kernel_times(mats, reps):
    """Duration per launch of each kernel (variant and shape), measured live with
    HIP events around each of `reps` graph replays that hold only that kernel's
    launches (at least 64, in step order): mean over the replays, and median and
    interquartile range of the per-replay figures.  Queued kernels start as the
    previous one ends, so elapsed time / launches is the kernel's own duration."""
    by = {}
    for m in mats:
        by.setdefault((variant_key(m), "%dx%d" % (m.N, m.K)), []).append(m)
    out = {}
    for (variant, shape), ms in by.items():
        n_step = len(ms)                  # launches of this kernel per step
        ms = with_copies(ms, 600 << 20)   # more distinct bytes than the caches hold
        rep = max(1, -(-64 // len(ms)))   # at least 64 launches per replay
        g = capture(ms * rep)
        ts = [t / (rep * len(ms)) for t in replay_times(g, reps, 2)]
        per_launch = float(np.mean(ts))
        med, iqr = quartiles(ts)
        out["%s %s" % (variant, shape)] = {
            "variant": variant, "shape": shape, "avg_s": per_launch, "median_s": med,
            "iqr_s": iqr, "launches": n_step, "bytes_per_launch": ms[0].bytes,
            "step_s": per_launch * n_step}
        del g, ms
    return out


def read_ceiling(nbytes, dev, reps):
    """What one kernel moving `nbytes` can reach here: lin_stream_read over a
    buffer of that size (a read-only pass with the products' launch shape),
    cycled over copies larger than the last-level cache and replayed
    back-to-back in a graph, like the products.  GB/s."""
    nbytes = max(16, nbytes // 16 * 16)
    copies = max(2, -(-(600 << 20) // nbytes))
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(copies)]
    n = max(32, 2 * copies)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(n):
            L.lin_stream_read(bufs[i % copies])
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(n):
            L.lin_stream_read(bufs[i % copies])
    _, gpu = time_graph(g, reps, 2)
    del g, bufs
    return nbytes / (gpu / n) / 1e9


def read_chain(mats, dev, reps, warmup):
    """The floor of a step launched one kernel per matrix: lin_stream_read over a
    buffer of each matrix's algorithmic bytes (weights, scales, x and y), one
    launch per matrix in step order, captured as one graph and replayed like the
    step.  Each launch is a read-only pass that does nothing else, so the chain's
    time is what the launches, their start ramps and their drains cost with no
    products at all.  Mean seconds per replay."""
    bufs = [torch.empty(max(16, m.bytes // 16 * 16), dtype=torch.uint8, device=dev) for m in mats]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for b in bufs:
            L.lin_stream_read(b)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for b in bufs:
            L.lin_stream_read(b)
    ts = replay_times(g, reps, warmup)
    del g, bufs
    return float(np.mean(ts))


def measured_traffic(key, shapes_mix):
    """HBM bytes per launch of kernel variant `key` over the step's shape mix,
    from the counter table, or None if none was taken for the current source."""
    import hashlib
    path = os.path.join(L.TUNING_DIR, "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        table = json.load(f)["measured"]
    for e in table:
        if e["kernel"] != key:
            continue
        src = b"".join(open(os.path.join(os.path.dirname(L.__file__), p), "rb").read()
                       for p in e["sources"])
        if hashlib.sha256(src).hexdigest()[:16] != e["src_sha256_16"]:
            return None
        tot, n = 0, 0
        for shape, count in shapes_mix.items():
            if shape not in e["per_shape"]:
                return None
            tot += count * (e["per_shape"][shape]["fetch_bytes"] + e["per_shape"][shape]["write_bytes"])
            n += count
        return int(tot / n)
    return None


# ---------------------------------------------------------------- batched tokens

MFMA_PEAK_TFS = 2500.0   # MI355X dense bf16 matrix-core peak


class SkinnyCase:
    """One batched-token product Y = X . W^T of a Mistral-7B-shaped matrix, bf16
    weights or int4-g64 weights in the tiled layout."""

    def __init__(self, M, N, K, fmt="bf16"):
        self.M, self.N, self.K, self.fmt = M, N, K, fmt
        self.bytes = bytes_bf16(N, K, M) if fmt == "bf16" else bytes_q4(N, K, M)
        self.flop = 2 * M * N * K
        self.kind = L.LIN_KIND_SKINNY_BF16 if fmt == "bf16" else L.LIN_KIND_SKINNY_Q4G64
        self.key = (self.kind, M, N, K)

    @property
    def name(self):
        return "M%d %dx%d" % (self.M, self.N, self.K)


def skinny_variant(c):
    cfg = L.lin_get_config(*c.key)
    if cfg["algo"] == L.LIN_ALGO_MFMA:
        return "mfma rows%d tm%d D%d S%d X%d%s" % (cfg["rows"], cfg["tile_m"], cfg["unroll"],
                                                  cfg["split"], cfg["stage_x"],
                                                  " W%d" % cfg["waves"] if cfg.get("waves") else "")
    return "valu R%d U%d S%d X%d tm%d" % (cfg["rows"], cfg["unroll"], cfg["split"],
                                         cfg["stage_x"], cfg["tile_m"])


def skinny_weights(N, K, fmt, copies, dev):
    """Distinct seeded weight copies of one shape: bf16 tensors, or int4-g64
    (quantised on the GPU) rearranged into the tiled layout at load."""
    out = []
    for i in range(copies):
        W = synth.weight(synth.MISTRAL_SEED, 0, N + i, N, K, device=dev)
        if fmt == "bf16":
            out.append(W)
        else:
            Wq, S = L.lin_quantize_q4g64(W)
            out.append(L.lin_q4g64_tile(Wq, S))
            del Wq, S, W
    torch.cuda.synchronize()
    return out


def run_skinny(args, dev, fmt):
    """Every (shape, M) product of the batched-decode workload: per case, a graph
    of back-to-back launches cycling over enough distinct weight copies to
    exceed the 256 MB last-level cache (so each launch streams W from HBM);
    the step is one launch of every case."""
    cases = [SkinnyCase(M, N, K, fmt) for M in synth.MISTRAL_M for N, K in synth.MISTRAL_SHAPES]
    tname = "mistral-7b-skinny.json" if fmt == "bf16" else "mistral-7b-skinny-q4.json"
    tfile = args.tuning or os.path.join(L.TUNING_DIR, tname)
    ok, stale = L.load_tuning(tfile) if (os.path.exists(tfile) and not args.tune) else ([], [])
    weights = {}
    for N, K in synth.MISTRAL_SHAPES:
        wbytes = 2 * N * K if fmt == "bf16" else bytes_q4(N, K, 0)
        copies = max(2, -(-(600 << 20) // wbytes))
        weights[(N, K)] = skinny_weights(N, K, fmt, copies, dev)
    X = {(M, K): synth.activation(synth.MISTRAL_SEED, 0, 0, M, K, device=dev)
         for M in synth.MISTRAL_M for K in {k for _, k in synth.MISTRAL_SHAPES}}
    Y = {c.key: torch.empty((c.M, c.N), dtype=torch.float32, device=dev) for c in cases}
    tuned = {}
    for c in cases:
        if c.key in ok:
            continue
        cfg = L.lin_autotune_set(c.kind, weights[(c.N, c.K)], X[(c.M, c.K)], Y[c.key])
        tuned[c.key] = cfg
        log("tuned skinny %-16s -> %s" % (c.name, cfg))
    if tuned:
        entries = {k: L.lin_get_config(*k) for k in (c.key for c in cases)}
        L.save_tuning(tfile, entries)
    tuning = "%s (%d cases, %d tuned now)" % (os.path.relpath(tfile, ROOT), len(cases), len(tuned))

    def graph_of(fn_list):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for f in fn_list:
                f()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for f in fn_list:
                f()
        torch.cuda.synchronize()
        return g

    def call(c, i):
        Wc = weights[(c.N, c.K)]
        fn = L.lin_gemm_skinny_bf16 if fmt == "bf16" else L.lin_gemm_skinny_q4g64
        return lambda: fn(Wc[i % len(Wc)], X[(c.M, c.K)], Y[c.key])

    reps = max(1, args.kernel_reps)
    per_case = {}
    for c in cases:
        n = max(32, 2 * len(weights[(c.N, c.K)]))
        g = graph_of([call(c, i) for i in range(n)])
        ts = [t / n for t in replay_times(g, reps, 2)]
        us = float(np.mean(ts)) * 1e6
        med, iqr = quartiles(ts)
        floor_us = max(c.bytes / (HBM_PEAK_GBS * 1e3), c.flop / (MFMA_PEAK_TFS * 1e6))
        per_case[c.name] = {"variant": skinny_variant(c), "us": round(us, 3),
                            "median_us": round(med * 1e6, 3), "iqr_us": round(iqr * 1e6, 3),
                            "GB_s": round(c.bytes / us / 1e3, 1),
                            "TFLOP_s": round(c.flop / us / 1e6, 1),
                            "hbm_frac": round(c.bytes / us / 1e3 / HBM_PEAK_GBS, 4),
                            "mfma_frac": round(c.flop / us / 1e6 / MFMA_PEAK_TFS, 4),
                            "roofline_time_frac": round(floor_us / us, 4),
                            "tok_s": round(c.M / us * 1e6, 1)}
        log("skinny %-16s %-34s %8.2f us %7.1f GB/s %6.1f TFLOP/s  %.0f%% of roofline time"
            % (c.name, per_case[c.name]["variant"], us, c.bytes / us / 1e3, c.flop / us / 1e6,
               100 * floor_us / us))
        del g
    step = graph_of([call(c, 0) for c in cases])
    wall, gpu = time_runs([step.replay], args.steps, args.warmup)
    step_bytes = sum(c.bytes for c in cases)
    dom = max(cases, key=lambda c: per_case[c.name]["us"])
    d = per_case[dom.name]
    ceil = read_ceiling(dom.bytes, dev, reps)
    # the roof that bounds the dominant case at peak specs: HBM bytes or MFMA FLOPs
    mfma_bound = dom.flop / (MFMA_PEAK_TFS * 1e6) > dom.bytes / (HBM_PEAK_GBS * 1e3)
    hbm = {"achieved": d["GB_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": d["hbm_frac"],
           "read_ceiling_GB_s": round(ceil, 1), "frac_of_read_ceiling": round(d["GB_s"] / ceil, 4)}
    mfma = {"achieved": d["TFLOP_s"], "peak": MFMA_PEAK_TFS, "unit": "TFLOP/s", "frac": d["mfma_frac"],
            "flop_per_launch": dom.flop}
    roofline = {"bound": "mfma" if mfma_bound else "hbm"}
    roofline.update(mfma if mfma_bound else hbm)
    roofline.update({"traffic": None, "kernel": d["variant"], "case": dom.name,
                     "avg_launch_us": d["us"], "bytes_per_launch": dom.bytes})
    roofline["hbm" if mfma_bound else "mfma"] = hbm if mfma_bound else mfma
    out = {"metric": METRIC, "value": round(step_bytes / wall / 1e9, 1), "unit": "GB/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(wall * 1e3, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None,
           "dtype": ("bf16 weights and tokens, fp32 accumulate" if fmt == "bf16" else
                     "int4-g64 weights (tiled at load), bf16 tokens, bf16 matrix-core products, "
                     "fp32 accumulate and scales"),
           "data": "synthetic",
           "config": {"workload": "mistral-7b-shaped batched-decode products%s, M in %s tokens x %d "
                      "shapes, one launch each per step" % ("" if fmt == "bf16" else ", int4-g64",
                                                          list(synth.MISTRAL_M),
                                                          len(synth.MISTRAL_SHAPES)),
                      "bytes_per_step": step_bytes, "tuning": tuning},
           "pct_of_hbm_peak": round(100.0 * step_bytes / wall / 1e9 / HBM_PEAK_GBS, 2),
           "gpu_ms_per_step": round(gpu * 1e3, 4), "cases": per_case, "roofline": roofline}
    if not args.skip_cpu:
        out["cpu_baseline"] = cpu_baseline_skinny(CPU_THREADS, fmt)
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------- fused epilogues

EPI_OF = {"o": L.LIN_EPI_ADD, "down": L.LIN_EPI_ADD, "gate|up": L.LIN_EPI_SWIGLU}


NORM_EPS = 1e-6


def _prepare(m, e, nrm):
    if e != L.LIN_EPI_NONE and not hasattr(m, "res"):
        n_out = m.N // 2 if e == L.LIN_EPI_SWIGLU else m.N
        m.res = torch.zeros((1, n_out), dtype=torch.float32, device=m.y.device)
        m.h = torch.empty((1, n_out), dtype=torch.float32, device=m.y.device)
    if nrm and not hasattr(m, "gain"):
        rng = np.random.default_rng(m.N * 131 + m.K)
        gbits = ((1.0 + 0.1 * rng.standard_normal(m.K)).astype(np.float32).view(np.uint32) >> 16)
        m.gain = synth.from_bits(gbits.astype(np.uint16), torch.bfloat16, m.y.device)
        m.xn = torch.empty_like(m.x)


def torch_rmsnorm(x, g, eps, out):
    """RMSNorm as separate PyTorch ops (the unfused reference pass)."""
    xf = x.float()
    out.copy_(xf * torch.rsqrt(xf.pow(2).mean(-1, keepdim=True) + eps) * g.float())


def fused_call(m, e, nrm):
    """One launch: the product with its epilogue and, if nrm, its RMSNorm prologue."""
    r = m.res if e == L.LIN_EPI_ADD else None
    y = m.y if e == L.LIN_EPI_NONE else m.h
    if nrm:
        if m.fmt == "bf16":
            return lambda: L.lin_gemv_bf16_norm(m.W, m.x, m.gain, NORM_EPS, e, r=r, y=y)
        if m.fmt == "i8":
            return lambda: L.lin_gemv_i8_norm(m.Wq, m.S, m.x, m.gain, NORM_EPS, e, r=r, y=y)
        return lambda: L.lin_gemv_q4g64_norm(m.Wq, m.S, m.x, m.gain, NORM_EPS, e, r=r, y=y)
    if e == L.LIN_EPI_NONE:
        return lambda: launch(m)
    if m.fmt == "bf16":
        return lambda: L.lin_gemv_bf16_ep(m.W, m.x, e, r=r, y=y)
    if m.fmt == "i8":
        return lambda: L.lin_gemv_i8_ep(m.Wq, m.S, m.x, e, r=r, y=y)
    return lambda: L.lin_gemv_q4g64_ep(m.Wq, m.S, m.x, e, r=r, y=y)


def epilogue_step(mats, fused, norms=False):
    """Launch list of one decode pass with the elementwise steps around the
    projections: the residual add after o and down, silu(gate) * up after
    gate|up and, with norms, the RMSNorm of the inputs of q|k|v, gate|up and
    the head.  fused: folded into the products (lin_gemv_*_ep, lin_gemv_*_norm);
    otherwise the plain product with separate PyTorch ops around it."""
    fns = []
    for m in mats:
        e = EPI_OF.get(m.name, L.LIN_EPI_NONE)
        nrm = norms and m.name in NORM_OF
        _prepare(m, e, nrm)
        if fused:
            fns.append(fused_call(m, e, nrm))
            continue
        if nrm:
            fns.append(lambda m=m: torch_rmsnorm(m.x, m.gain, NORM_EPS, m.xn))
            if m.fmt == "bf16":
                fns.append(lambda m=m: L.lin_gemv_bf16(m.W, m.xn, m.y))
            elif m.fmt == "i8":
                fns.append(lambda m=m: L.lin_gemv_i8(m.Wq, m.S, m.xn, m.y))
            else:
                fns.append(lambda m=m: L.lin_gemv_q4g64(m.Wq, m.S, m.xn, m.y))
        else:
            fns.append(lambda m=m: launch(m))
        if e == L.LIN_EPI_ADD:
            fns.append(lambda m=m: torch.add(m.y, m.res, out=m.h))
        elif e == L.LIN_EPI_SWIGLU:
            half = m.N // 2
            fns.append(lambda m=m, half=half: torch.mul(torch.nn.functional.silu(m.y[:, :half]),
                                                        m.y[:, half:], out=m.h))
    return fns


def prologue_cost(mats, args):
    """Per normalised projection shape: average launch time of the product with
    its epilogue, without and with the RMSNorm prologue (graphs of back-to-back
    launches over every matrix of that shape, as the step runs them)."""
    out = {}
    for name in NORM_OF:
        ms = [m for m in mats if m.name == name]
        if not ms:
            continue
        e = EPI_OF.get(name, L.LIN_EPI_NONE)
        reps = max(1, 64 // len(ms))
        res = {}
        for nrm in (False, True):
            for m in ms:
                _prepare(m, e, nrm)
            g = capture_fns([fused_call(m, e, nrm) for _ in range(reps) for m in ms])
            _, gpu = time_graph(g, max(5, args.steps // 2), args.warmup)
            res["norm" if nrm else "plain"] = gpu / (reps * len(ms))
            del g
        out["%s %dx%d" % (name, ms[0].N, ms[0].K)] = {
            "us_without": round(res["plain"] * 1e6, 3), "us_with_norm": round(res["norm"] * 1e6, 3),
            "GB_s_with_norm": round(ms[0].bytes / res["norm"] / 1e9, 1)}
    return out


def capture_fns(fns):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for f in fns:
            f()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    torch.cuda.synchronize()
    return g


def run_epilogues(sets, fmts, args):
    """Fused against unfused decode passes (epilogues only, then epilogues and
    RMSNorm prologues), and the per-kernel cost of the prologue; per format."""
    out = {}
    for f in fmts:
        res = {}
        for norms in (False, True):
            part = {}
            for fused in (False, True):
                fns = epilogue_step(sets[f], fused, norms)
                g = capture_fns(fns)
                _, gpu = time_graph(g, max(5, args.steps // 2), args.warmup)
                part["fused" if fused else "unfused"] = {"launches": len(fns),
                                                         "us_per_token": round(gpu * 1e6, 2)}
                del g
            part["speedup"] = round(part["unfused"]["us_per_token"] / part["fused"]["us_per_token"], 4)
            log("%s %s: unfused %.1f us (%d launches), fused %.1f us (%d launches)"
                % ("epilogues+norms" if norms else "epilogues", f, part["unfused"]["us_per_token"],
                   part["unfused"]["launches"], part["fused"]["us_per_token"],
                   part["fused"]["launches"]))
            if norms:
                res["with_norms"] = part
            else:
                res.update(part)
        res["prologue_cost"] = prologue_cost(sets[f], args)
        for k, v in res["prologue_cost"].items():
            log("prologue %s %s: %.2f -> %.2f us" % (f, k, v["us_without"], v["us_with_norm"]))
        out[f] = res
    return out


# ---------------------------------------------------------------- CPU baseline

def cpu_baseline(model, layers, threads, fmts=("bf16", "q4")):
    """The oracle, as it stands, on the host cores: a bounded sample (the first
    `layers` layers, in the same formats), rows split over `threads` threads;
    then one thread over the attention projections of layer 0."""
    import oracle
    work = []
    for layer, idx, name, N, K in synth.decode_matrices(model):
        if layer >= layers:
            continue
        W = synth.bits(synth.weight(model["seed"], layer, idx, N, K))
        x = synth.bits(synth.activation(model["seed"], layer, idx, 1, K))
        if "bf16" in fmts:
            work.append(("bf16", W, None, x, bytes_bf16(N, K), layer, name))
        if "q4" in fmts:
            Wq, S = oracle.quantize_q4g64(W)
            work.append(("q4", Wq, S, x, bytes_q4(N, K), layer, name))
        if "i8" in fmts:
            Wq, S = oracle.quantize_i8(W)
            work.append(("i8", Wq, S, x, bytes_i8(N, K), layer, name))
    total_bytes = sum(w[4] for w in work)

    def run_rows(item, lo, hi):
        fmt, A, S, x = item[:4]
        if fmt == "bf16":
            oracle.gemm_dense(A[lo:hi], x)
        elif fmt == "q4":
            oracle.gemm_q4g64(A[lo:hi], S[lo:hi], x)
        else:
            oracle.gemm_i8(A[lo:hi], S[lo:hi], x)

    def timed(items, nthreads):
        jobs = []
        for item in items:
            N = item[1].shape[0]
            step = max(1, N // (4 * nthreads))
            jobs += [(item, lo, min(N, lo + step)) for lo in range(0, N, step)]
        t0 = time.perf_counter()
        with concurrent.futures.ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(lambda j: run_rows(*j), jobs))
        return time.perf_counter() - t0

    dt = timed(work, threads)
    # one thread on the attention projections of layer 0 (a shorter sample)
    first = [w for w in work if w[5] == 0 and w[6] in ("q", "k", "v", "o")]
    dt1 = timed(first, 1)
    b1 = sum(w[4] for w in first)
    step_bytes = sum((bytes_bf16 if f == "bf16" else bytes_q4 if f == "q4" else bytes_i8)(N, K)
                     for f in fmts for _, _, _, N, K in synth.decode_matrices(model))
    gbs = total_bytes / dt / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": threads,
            "host_cores": os.cpu_count(),
            "kind": "oracle",
            "sample": "%s layers 0-%d (%d matrices), %s, %.1f MB of weights, "
                      "batch 1, fp64 sequential sums, %d threads, %.2f s wall"
                      % (model["name"], layers - 1, len(work) // len(fmts),
                         " and ".join(FORMAT_NAMES[f] for f in fmts), total_bytes / 1e6,
                         threads, dt),
            "s_per_step_extrapolated": round(step_bytes / (gbs * 1e9), 3),
            "equiv_tok_s_extrapolated": round(gbs * 1e9 / step_bytes, 4),
            "one_thread": {"value": round(b1 / dt1 / 1e9, 4), "unit": "GB/s",
                           "sample": "layer 0 q, k, v, o (%d matrices), %.1f MB, %.2f s wall"
                                     % (len(first) // len(fmts), b1 / 1e6, dt1)},
            "cpu_model": cpu_model()}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_skinny(threads, fmt="bf16", rows=96):
    """The oracle on a bounded sample of the batched workload: the first `rows`
    rows of every shape against all M tokens, for every M."""
    import oracle
    work = []
    for M in synth.MISTRAL_M:
        for N, K in synth.MISTRAL_SHAPES:
            W = synth.bits(synth.weight(synth.MISTRAL_SEED, 0, N, N, K)[:rows])
            Xb = synth.bits(synth.activation(synth.MISTRAL_SEED, 0, 0, M, K))
            if fmt == "bf16":
                work.append(((W,), Xb, bytes_bf16(rows, K, M)))
            else:
                work.append((oracle.quantize_q4g64(W), Xb, bytes_q4(rows, K, M)))
    total = sum(w[2] for w in work)
    jobs = [(tuple(a[lo:lo + 8] for a in Ws), Xb) for Ws, Xb, _ in work
            for lo in range(0, rows, 8)]
    fn = oracle.gemm_dense if fmt == "bf16" else oracle.gemm_q4g64
    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda j: fn(*j[0], j[1]), jobs))
    dt = time.perf_counter() - t0
    return {"value": round(total / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "host_cores": os.cpu_count(), "kind": "oracle",
            "sample": "first %d rows of each of the %d shapes x M in %s, fp64 sequential sums, "
                      "%.2f s wall" % (rows, len(synth.MISTRAL_SHAPES), list(synth.MISTRAL_M), dt)}


# ---------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen7b",
                    choices=["tinyllama", "qwen7b", "mistral-skinny", "mistral-skinny-q4"])
    ap.add_argument("--tune", action="store_true",
                    help="re-run lin_autotune for every shape and rewrite the tuning table")
    ap.add_argument("--tuning", default=None, help="tuning table path")
    ap.add_argument("--formats", default="bf16,q4",
                    help="weight formats of the decode-step workloads, in step order: any of "
                         "bf16, q4 (int4-g64), i8 (INT8, fp32 scale per row)")
    ap.add_argument("--epilogues", action="store_true",
                    help="also time decode passes with the residual adds and the gated silu "
                         "product (and then also the RMSNorm of the projection inputs), fused "
                         "into the products against separate PyTorch ops")
    ap.add_argument("--kernel-reps", type=int, default=30, metavar="N",
                    help="graph replays per kernel variant for the per-kernel timings (default 30; "
                         "counter passes under a profiler use 1)")
    ap.add_argument("--save-tuning", default=None, metavar="PATH",
                    help="write the tuning table, with any entries tuned by this run, to PATH")
    ap.add_argument("--no-fuse", action="store_true",
                    help="one launch per matrix instead of q|k|v and gate|up concatenated")
    ap.add_argument("--cpu-layers", type=int, default=None,
                    help="layers in the oracle's timed sample (default: 8 for qwen7b, 16 for "
                         "tinyllama)")
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--counter-pass", action="store_true",
                    help="only launch every matrix of the decode step once, eagerly and in step "
                         "order, twice over (the dispatches a profiler's HBM byte counters are "
                         "read from), print the launch list and exit")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES three times (scales the HBM "
                         "byte counters of a profiler run) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the decode-step linear layer is built and timed on a "
              "single MI355X; --gpus %d is not supported." % args.gpus, file=sys.stderr)
        sys.exit(2)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = args.copy_calibration
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": 3}), flush=True)
        return
    if args.workload in ("mistral-skinny", "mistral-skinny-q4"):
        run_skinny(args, dev, "bf16" if args.workload == "mistral-skinny" else "q4")
        return
    model = synth.TINYLLAMA if args.workload == "tinyllama" else synth.QWEN7B
    log("building %s weight sets on %s" % (model["name"], torch.cuda.get_device_name(dev)))
    fused = not args.no_fuse
    fmts = [f.strip() for f in args.formats.split(",") if f.strip()]
    if not fmts or any(f not in KINDS for f in fmts) or len(set(fmts)) != len(fmts):
        print("--formats takes distinct entries of bf16, q4, i8", file=sys.stderr)
        sys.exit(2)
    sets = {f: build_set(model, f, dev, fused) for f in fmts}
    allm = [m for f in fmts for m in sets[f]]
    default_fmts = fmts == ["bf16", "q4"]
    tname = model["name"] + ("" if default_fmts else "-" + "-".join(fmts))
    tfile = args.tuning or os.path.join(L.TUNING_DIR, "%s.json" % tname)
    tuning = apply_tuning(allm, tfile, args.tune, norms=args.epilogues, save_to=args.save_tuning)
    log("tuning: " + tuning)
    if args.counter_pass:
        counter_pass(allm)
        return

    step_bytes = sum(m.bytes for m in allm)
    fmt_bytes = {f: sum(m.bytes for m in sets[f]) for f in sets}

    # one kernel per (fused) matrix, each format's step captured as one graph
    graphs = {f: capture(sets[f]) for f in sets}
    per_fmt = {}
    for f in fmts:
        ts = replay_times(graphs[f], max(30, args.steps), args.warmup)
        gpu_f = float(np.mean(ts))
        med, iqr = quartiles(ts)
        # the same pass without the graph: one host call per matrix
        eager, _ = time_runs([lambda f=f: [launch(m) for m in sets[f]]], max(10, args.steps // 2),
                             args.warmup)
        chain = read_chain(sets[f], dev, max(30, args.steps), args.warmup)
        per_fmt[f] = {"ms_per_token": round(gpu_f * 1e3, 4), "equiv_tok_s": round(1.0 / gpu_f, 1),
                      "GB_s": round(fmt_bytes[f] / gpu_f / 1e9, 1), "bytes": fmt_bytes[f],
                      "median_ms": round(med * 1e3, 4), "iqr_ms": round(iqr * 1e3, 4),
                      "no_graph_ms_per_token": round(eager * 1e3, 4),
                      "read_chain_ms": round(chain * 1e3, 4),
                      "read_chain_GB_s": round(fmt_bytes[f] / chain / 1e9, 1),
                      "frac_of_read_chain": round(chain / gpu_f, 4)}
        log("%s step: %.1f us (median %.1f, IQR %.1f), %.1f GB/s, %.0f tok/s; without the graph "
            "%.1f us; read chain %.1f us" % (f, gpu_f * 1e6, med * 1e6, iqr * 1e6,
                                             fmt_bytes[f] / gpu_f / 1e9, 1 / gpu_f, eager * 1e6,
                                             chain * 1e6))
    # the timed region: K steps of the whole path (one decode pass per format, in
    # order), the step captured as one graph like each format's pass
    step_graph = capture(allm)
    warm(step_graph)
    torch.cuda.synchronize()
    wall, gpu = time_runs([step_graph.replay], args.steps, args.warmup)
    gbs = step_bytes / wall / 1e9
    del step_graph

    kt = kernel_times(allm, reps=args.kernel_reps)
    dom_key = max(kt, key=lambda k: kt[k]["step_s"])
    dom = kt[dom_key]
    achieved = dom["bytes_per_launch"] / dom["avg_s"] / 1e9
    ceil = {k: read_ceiling(v["bytes_per_launch"], dev, max(1, min(5, args.kernel_reps)))
            for k, v in kt.items()}
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(dom["variant"], {dom["shape"]: 1}),
                "read_ceiling_GB_s": round(ceil[dom_key], 1),
                "frac_of_read_ceiling": round(achieved / ceil[dom_key], 4),
                "kernel": dom["variant"], "shape": dom["shape"],
                "launches_per_step": dom["launches"],
                "avg_launch_us": round(dom["avg_s"] * 1e6, 3),
                "bytes_per_launch": int(dom["bytes_per_launch"]),
                "share_of_step": round(dom["step_s"] / gpu, 3)}
    kernels = {k: {"avg_us": round(v["avg_s"] * 1e6, 3), "median_us": round(v["median_s"] * 1e6, 3),
                   "iqr_us": round(v["iqr_s"] * 1e6, 3), "launches": v["launches"],
                   "GB_s": round(v["bytes_per_launch"] / v["avg_s"] / 1e9, 1),
                   "read_ceiling_GB_s": round(ceil[k], 1),
                   "algorithmic_bytes": int(v["bytes_per_launch"]),
                   "traffic": measured_traffic(v["variant"], {v["shape"]: 1})}
               for k, v in sorted(kt.items(), key=lambda kv: -kv[1]["step_s"])}

    out = {"metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "%s weights, bf16 x, fp32 accumulate" % " and ".join(FORMAT_NAMES[f] for f in fmts),
           "data": "synthetic",
           "config": {"workload": "%s decode weight set, batch 1, %s (%d matrices "
                      "each%s)" % (model["name"], " + ".join(FORMAT_NAMES[f] for f in fmts),
                                   len(synth.decode_groups(model, False)),
                                   ", q|k|v and gate|up concatenated at load" if fused else ""),
                      "batch": 1, "launches_per_step": len(allm), "bytes_per_step": step_bytes,
                      "fused_projections": fused, "tuning": tuning},
           "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
           "gpu_ms_per_step": round(gpu * 1e3, 4),
           "per_format": per_fmt, "kernels": kernels, "roofline": roofline}
    # context: what a plain read of 4 GB reaches on this part (not the metric's denominator)
    big = read_ceiling(4 << 30, dev, max(1, min(5, args.kernel_reps)))
    out["achievable_read"] = {"bytes": 4 << 30, "GB_s": round(big, 1),
                              "frac_of_peak": round(big / HBM_PEAK_GBS, 4)}
    if args.epilogues:
        if not fused:
            print("--epilogues needs the concatenated gate|up projections (no --no-fuse)", file=sys.stderr)
            sys.exit(2)
        out["epilogues"] = run_epilogues(sets, fmts, args)
    if not args.skip_cpu:
        layers = args.cpu_layers or (16 if model is synth.TINYLLAMA else 8)
        out["cpu_baseline"] = cpu_baseline(model, layers, CPU_THREADS, fmts)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
