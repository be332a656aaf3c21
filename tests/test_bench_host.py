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


def test_host_info_names_the_cpu():
    h = bench.host_info()
    assert h["nproc"] >= 1 and h["affinity_cpus"] >= 1
    assert h["cpu_model"]


def test_cpu_oracle_is_built_for_this_host_and_timed():
    """The CPU baseline's oracle: a native -O3 build of the same oracle.c,
    giving the same numbers as the portable build the tests use."""
    import numpy as np
    import oracle
    import synth
    orc = bench.CpuOracle(bench.host_info())
    assert orc.threads >= 1
    w = synth.WORKLOADS["prefill_hq4_hkv2_d32_m16"]
    q, k, v = synth.prefill_inputs(w)
    args = (q, k, v, w.m, w.q_stride, w.kv_stride, w.num_q_heads, w.heads_per_kv, w.head_dim)
    out, ts = orc.time(lambda: orc.o.prefill_causal(*args), reps=3)
    assert len(ts) >= 3 and min(ts) > 0
    ref = oracle.prefill_causal(*args)
    # both builds evaluate every sum in the same order without contraction
    assert np.array_equal(out, ref)
    rec = orc.record(w.flops(), 1e9, "GFLOP/s", ts, "test")
    assert rec["kind"] == "oracle" and rec["cores"] == orc.threads and rec["value"] > 0
    assert rec["cpu_model"] and rec["nproc"] >= 1


def test_parity_bound():
    import numpy as np
    ref = np.array([1.0, -2.0, 3.0])
    p = bench.parity(np.array([1.0, -2.0, 3.0], np.float32), ref, 4.0)
    assert p["ok"] and p["max_abs_err"] == 0.0
    p = bench.parity(np.array([1.0, -2.0, 3.001], np.float32), ref, 4.0)
    assert not p["ok"] and p["bound"] == bench.TOL * 4.0
