"""The summariser of rocprofv3 kernel traces of bench.py runs: each step kernel's
dispatches are found by kernel instance and by the grid its shape launches, on
small hand-written CSVs."""
import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SCRIPT = os.path.join(ROOT, "memory_bound_weight_amd", "tuning", "trace_summary.py")
BF16 = "void lin::gemv_bf16_valu<1, 1, 7, 1, false, 0, false>(lin::KArgs)"
XRES = "void lin::gemv_q4_xres<1, 2, 8, 10, 0>(lin::KArgs)"


def _write(tmp_path, dispatches, kernels):
    t = str(tmp_path)
    with open(t + "/run_kernel_stats.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs",
                                          "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writeheader()
        w.writerow({"Name": BF16, "Calls": 3, "TotalDurationNs": 30000, "AverageNs": 10000,
                    "Percentage": 60.0, "MinNs": 9000, "MaxNs": 11000, "StdDev": 0})
    with open(t + "/run_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z",
                                          "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        t0 = 0
        for name, grid, ns in dispatches:
            w.writerow({"Kernel_Name": name, "Grid_Size_X": grid, "Grid_Size_Y": 1,
                        "Grid_Size_Z": 1, "Start_Timestamp": t0, "End_Timestamp": t0 + ns})
            t0 += ns + 100
    with open(t + "/bench.log", "w") as f:
        f.write("building\n" + json.dumps({"value": 1.0, "kernels": kernels}) + "\n")
    r = subprocess.run([sys.executable, SCRIPT, "--trace", t + "/run", "--bench", t + "/bench.log",
                        "--out", t + "/out.md", "--reduced", t + "/red.csv"],
                       capture_output=True, text=True)
    return r, open(t + "/out.md").read() if r.returncode == 0 else ""


def test_dispatches_are_matched_by_instance_and_grid(tmp_path):
    # bf16 R1 U7 S1: four rows per workgroup -> 4608 rows = 1152 workgroups;
    # int4 x-resident R10 S2: 20 rows per workgroup -> 231, rounded up to 256
    bf_grid, q4_grid = 1152 * 256, 256 * 256
    disp = [(BF16, bf_grid, 6000), (BF16, bf_grid, 8000), (BF16, 1024 * 256, 50000),
            (XRES, q4_grid, 4000), (XRES, 999 * 256, 90000)]
    kernels = {"gemv_bf16 R1 U7 S1 X0 4608x3584": {"avg_us": 7.0, "launches": 28},
               "gemv_q4g64 R10 U8 S2 X2 4608x3584": {"avg_us": 4.0, "launches": 28}}
    r, md = _write(tmp_path, disp, kernels)
    assert r.returncode == 0, r.stderr
    rows = {ln.split("|")[1].strip(): [c.strip() for c in ln.split("|")]
            for ln in md.splitlines() if ln.startswith("| `gemv")}
    bf = rows["`gemv_bf16 R1 U7 S1 X0`"]
    assert bf[5] == "2" and bf[6] == "7.00" and bf[9] == "0.0 %"   # the two 1152-workgroup dispatches
    q4 = rows["`gemv_q4g64 R10 U8 S2 X2`"]
    assert q4[5] == "1" and q4[6] == "4.00"
    red = list(csv.DictReader(open(str(tmp_path) + "/red.csv")))
    assert {(x["grid_items"], x["dispatches"]) for x in red} >= {(str(bf_grid), "2"), (str(q4_grid), "1")}


def test_unmatched_shape_is_reported_not_guessed(tmp_path):
    disp = [(BF16, 1000 * 256, 6000)]
    kernels = {"gemv_bf16 R1 U7 S1 X0 4608x3584": {"avg_us": 7.0, "launches": 28}}
    r, md = _write(tmp_path, disp, kernels)
    assert r.returncode == 0, r.stderr
    assert "(0 matching instances at grid 294912)" in md


def test_shapes_sharing_instance_and_grid_are_flagged(tmp_path):
    # o 2048x2048 and down 2048x5632 with one variant: same N, same grid
    grid = 512 * 256
    bf = "void lin::gemv_bf16_valu<1, 1, 4, 1, false, 0, false>(lin::KArgs)"
    disp = [(bf, grid, 3000), (bf, grid, 5000)]
    kernels = {"gemv_bf16 R1 U4 S1 X0 2048x2048": {"avg_us": 3.0, "launches": 22},
               "gemv_bf16 R1 U4 S1 X0 2048x5632": {"avg_us": 5.0, "launches": 22}}
    r, md = _write(tmp_path, disp, kernels)
    assert r.returncode == 0, r.stderr
    assert "(traced with 2048x5632: same instance and grid)" in md
    assert "(traced with 2048x2048: same instance and grid)" in md
