"""The converter from rocprofv3 counter CSVs to the HBM traffic table that
bench.py reports beside each kernel's algorithmic bytes: copy calibration, the
pairing of the last counter pass with the launch list, and per-shape medians,
on small hand-written CSVs."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SCRIPT = os.path.join(ROOT, "memory_bound_weight_amd", "tuning", "hbm_counters.py")
COLS = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
GEMV = "void lin::gemv_bf16_valu<1, 1, 2, 4, false, 0, false>(lin::KArgs)"
XRES = "void lin::gemv_q4_xres<1, 2, 4, 4, 0>(lin::KArgs)"


def _csv(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "pmc_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COLS)
        w.writeheader()
        for i, (name, v) in enumerate(rows, 1):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Grid_Size": 256,
                        "Counter_Name": counter, "Counter_Value": v})


def _run(tmp_path, fetch, write, seq):
    t = str(tmp_path)
    _csv(t + "/f", "FETCH_SIZE", fetch)
    _csv(t + "/w", "WRITE_SIZE", write)
    # a 1 MiB copy that counts half its reads and all its writes
    _csv(t + "/cf", "FETCH_SIZE", [("fill", 1024.0), ("__amd_rocclr_copyBuffer", 512.0)])
    _csv(t + "/cw", "WRITE_SIZE", [("fill", 1024.0), ("__amd_rocclr_copyBuffer", 1024.0)])
    with open(t + "/log", "w") as f:
        f.write("building\n" + json.dumps({"counter_pass": seq, "passes": 2}) + "\n")
    out = t + "/table.json"
    r = subprocess.run([sys.executable, SCRIPT, "--fetch", t + "/f", "--write", t + "/w",
                        "--copy-fetch", t + "/cf", "--copy-write", t + "/cw",
                        "--copy-bytes", str(1 << 20), "--launches", t + "/log", "--out", out],
                       capture_output=True, text=True)
    return r, out


def test_last_pass_is_paired_in_order_and_scaled(tmp_path):
    seq = [["gemv_bf16 R1 U2 S4 X0", "64x64"], ["gemv_q4g64 R4 U4 S2 X2", "64x64"],
           ["gemv_bf16 R1 U2 S4 X0", "64x64"]]
    # weight generation, then two passes; only the second pass counts
    fetch = [("fill", 9.0)] + [(GEMV, 100.0), (XRES, 100.0), (GEMV, 100.0)] + \
            [(GEMV, 10.0), (XRES, 4.0), (GEMV, 30.0)]
    write = [("fill", 9.0)] + [(GEMV, 100.0), (XRES, 100.0), (GEMV, 100.0)] + \
            [(GEMV, 1.0), (XRES, 2.0), (GEMV, 1.0)]
    r, out = _run(tmp_path, fetch, write, seq)
    assert r.returncode == 0, r.stderr
    t = {e["kernel"]: e for e in json.load(open(out))["measured"]}
    bf = t["gemv_bf16 R1 U2 S4 X0"]
    assert bf["fetch_scale"] == 2.0 and bf["write_scale"] == 1.0
    assert bf["function"] == "gemv_bf16_valu"
    # median of the two bf16 launches (10 and 30 KiB, times 2)
    assert bf["per_shape"]["64x64"] == {"fetch_bytes": 40960, "write_bytes": 1024, "dispatches": 2}
    q4 = t["gemv_q4g64 R4 U4 S2 X2"]
    assert q4["function"] == "gemv_q4_xres"
    assert q4["per_shape"]["64x64"]["fetch_bytes"] == 8192
    assert q4["sources"][0] == "csrc/gemv_q4x.hip"


def test_misaligned_launch_list_is_refused(tmp_path):
    seq = [["gemv_bf16 R1 U2 S4 X0", "64x64"], ["gemv_q4g64 R4 U4 S2 X2", "64x64"]]
    # the dispatches come in the other order than the launch list says
    fetch = [(XRES, 1.0), (GEMV, 1.0), (XRES, 1.0), (GEMV, 1.0)]
    r, _ = _run(tmp_path, fetch, fetch, seq)
    assert r.returncode != 0 and "do not line up" in (r.stderr + r.stdout)


def test_one_pass_only_is_refused(tmp_path):
    seq = [["gemv_bf16 R1 U2 S4 X0", "64x64"]]
    r, _ = _run(tmp_path, [(GEMV, 1.0)], [(GEMV, 1.0)], seq)
    assert r.returncode != 0 and "two passes" in (r.stderr + r.stdout)
