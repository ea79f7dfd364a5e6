"""Host logic of bench.py that needs no GPU: the traffic figure is taken only
from a counter profile of the current gate source, and runs on more than one
GPU are refused with a message."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_traffic_needs_matching_source(tmp_path, monkeypatch):
    sha = bench.source_sha(bench.GATE_SOURCE)
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps({"w": {"gate_source_sha": sha, "hbm_bytes_per_launch": 123.0},
                             "stale": {"gate_source_sha": "0" * 16, "hbm_bytes_per_launch": 1.0}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.gate_traffic("w", 0.0) == 123.0
    assert bench.gate_traffic("stale", 0.0) is None
    assert bench.gate_traffic("absent", 0.0) is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.gate_traffic("w", 0.0) is None


def test_committed_profile_covers_default_workload():
    with open(bench.TRAFFIC_FILE) as fh:
        t = json.load(fh)
    entry = t["kimi-k2-prefill"]
    assert entry["hbm_bytes_per_launch"] > entry["algorithmic_bytes"] * 0.9
    assert entry["fetch_bytes"] > 0 and entry["write_bytes"] > 0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "single MI355X" in r.stderr and r.stdout == ""
