"""bench.py on the CPU: the one-GPU contract of the command line, and the
lookup of measured HBM traffic (reported only while the kernel sources match
the hash the counters were taken for)."""
import json
import os
import subprocess
import sys

import pytest

import bench
import memory_bound_weight_amd as L
sys.path.insert(0, os.path.join(os.path.dirname(L.__file__), "tuning"))
import hbm_counters  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv,
                       env=dict(os.environ, **env), capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single MI355X" in r.stderr


def _table(tmp_path, variant, shape, fetch, write, digest=None):
    srcs = hbm_counters.sources(variant)
    e = {"kernel": variant, "sources": srcs,
         "src_sha256_16": digest or hbm_counters.source_hash(srcs),
         "per_shape": {shape: {"fetch_bytes": fetch, "write_bytes": write}}}
    with open(tmp_path / "hbm_traffic.json", "w") as f:
        json.dump({"measured": [e]}, f)


def test_traffic_is_reported_for_matching_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(L, "TUNING_DIR", str(tmp_path))
    _table(tmp_path, "gemv_bf16 R1 U2 S4 X0", "64x64", 1000, 24)
    assert bench.measured_traffic("gemv_bf16 R1 U2 S4 X0", {"64x64": 1}) == 1024
    assert bench.measured_traffic("gemv_bf16 R1 U2 S4 X0", {"128x64": 1}) is None   # no such shape
    assert bench.measured_traffic("gemv_bf16 R2 U2 S4 X0", {"64x64": 1}) is None    # no such variant


def test_traffic_is_withheld_once_the_sources_change(tmp_path, monkeypatch):
    monkeypatch.setattr(L, "TUNING_DIR", str(tmp_path))
    _table(tmp_path, "gemv_q4g64 R4 U4 S2 X2", "64x64", 1000, 24, digest="0000000000000000")
    assert bench.measured_traffic("gemv_q4g64 R4 U4 S2 X2", {"64x64": 1}) is None

