"""Host-side checks of bench.py that need no GPU: the HBM-traffic figure is
read from the committed rocprofv3 summary only while that summary was taken
on the current kernel source, and multi-GPU runs are refused."""

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_traffic_summary_parses_when_source_matches(monkeypatch):
    kv = {}
    for line in open(bench.TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    monkeypatch.setattr(bench, "source_digest", lambda: kv["source_sha256"])
    t = bench.recorded_traffic(kv["workload"])
    assert t == float(kv["traffic_bytes_per_launch"])
    assert t > 0


def test_traffic_is_null_for_other_source_or_workload(monkeypatch):
    monkeypatch.setattr(bench, "source_digest", lambda: "0" * 64)
    assert bench.recorded_traffic(bench.DEFAULT_WORKLOAD) is None
    monkeypatch.undo()
    assert bench.recorded_traffic("no_such_workload") is None


def test_multi_gpu_request_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
