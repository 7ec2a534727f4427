"""Host-side checks of bench.py: the oracle baseline, the one-GPU guard and the traffic record check."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def test_cpu_baseline_samples_whole_heads():
    wl = workloads.workload("tiny")
    r = bench.cpu_baseline(wl, 60.0)  # the tiny layer finishes well within the budget
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s"
    assert r["value"] > 0 and r["cores"] >= 1
    n_heads = wl.batch * wl.heads
    assert f"{n_heads} of {n_heads} heads" in r["sample"]
    assert f"{n_heads * wl.n_cubes} query cubes in all" in r["sample"]


def test_cpu_baseline_stops_at_budget():
    wl = workloads.workload("tiny")
    r = bench.cpu_baseline(wl, 0.0)  # stops after the first query cube
    assert "1 query cubes in all" in r["sample"] and r["value"] > 0


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr


def test_traffic_record_needs_matching_sources(tmp_path, monkeypatch):
    rec = {"kernel_sha256_16": "0" * 16, "hbm_bytes_per_launch": 123}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "attn_fwd_wan1.3b_traffic.txt").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda kernel="attn_fwd": "f" * 16)
    assert bench.measured_traffic("wan1.3b") is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda kernel="attn_fwd": "0" * 16)
    assert bench.measured_traffic("wan1.3b") == 123


if __name__ == "__main__":
    sys.exit(pytest.main([__file__, "-q"]))
