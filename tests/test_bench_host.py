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



def test_percentiles_and_host_facts():
    xs = [5.0, 1.0, 3.0, 2.0, 4.0]
    assert bench.pct(xs, 50) == 3.0 and bench.pct(xs, 0) == 1.0 and bench.pct(xs, 100) == 5.0
    assert abs(bench.pct(xs, 10) - 1.4) < 1e-12
    h = bench.host_facts(7)
    assert h["os_cpu_count"] == os.cpu_count() and h["blas_threads"] == 7
    assert h["cpu_model"]


def test_family_roofline_is_mean_work_over_mean_time():
    class Op:
        def __init__(self, kind, flops=0, nbytes=0):
            self.kind, self.flops, self.bytes = kind, flops, nbytes

    class HP:
        ops = [Op("gemm", flops=2e12), Op("quant", nbytes=4e9), Op("gemm", flops=4e12),
               Op("weight_quant", nbytes=2e9)]

    mean_us = {0: 1000.0, 1: 1000.0, 2: 3000.0, 3: 500.0}
    r = bench.family_roofline(HP, mean_us, ("gemm",), "flops")
    assert r["achieved"] == 1500.0 and r["frac"] == 0.3 and r["launches_per_step"] == 2
    q = bench.family_roofline(HP, mean_us, ("quant", "weight_quant"), "bytes")
    # 3e9 bytes per launch over 750 us
    assert q["achieved"] == 4000.0 and q["frac"] == 0.5 and q["unit"] == "GB/s"
