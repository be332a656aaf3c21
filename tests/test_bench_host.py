"""Host-side rules of bench.py (CPU only): the one-GPU restriction and the
digest gate on stored HBM traffic counters."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                          capture_output=True, text=True, timeout=120)
    assert proc.returncode == 2
    assert "one GPU" in proc.stderr
    assert proc.stdout == ""  # no JSON line for an unsupported run


def test_source_digest_is_stable_hex():
    d = bench.source_digest()
    assert len(d) == 16 and int(d, 16) >= 0
    assert bench.source_digest() == d


def test_traffic_is_reported_only_for_the_measured_sources(tmp_path, monkeypatch):
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps({
        "k_now": {"source_digest": bench.source_digest(), "bytes_per_launch": 123},
        "k_old": {"source_digest": "0" * 16, "bytes_per_launch": 456}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.measured_traffic("k_now") == 123
    assert bench.measured_traffic("k_old") is None   # counters of other kernel sources
    assert bench.measured_traffic("missing") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.json"))
    assert bench.measured_traffic("k_now") is None
