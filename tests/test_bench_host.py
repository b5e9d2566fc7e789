"""Host-side logic of bench.py that needs no GPU: the one-GPU guard and the
rule that the committed HBM-traffic figure is reported only for the GEMM
source it was measured on."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_only_for_the_measured_source(tmp_path, monkeypatch):
    rec = {"gemm_source_sha256_16": bench.gemm_source_hash(), "hbm_bytes_per_launch": 123}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.load_traffic() == 123
    rec["gemm_source_sha256_16"] = "0" * 16         # measured on another source
    f.write_text(json.dumps(rec))
    assert bench.load_traffic() is None
    f.write_text("not json")
    assert bench.load_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.load_traffic() is None

