"""bench.py end to end on the tiny workload: every optional leg runs and the
JSON line carries the fields its contract names (the headline, both
rooflines, the cold sweep with the copy ceiling, the vendor comparison, the
graph replay, the clock window, the scale-format accuracy and the oracle
baseline)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line_on_tiny_workload_with_every_leg():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny_256x512x384",
           "--steps", "3", "--warmup", "1", "--reps", "5", "--clock-window", "0.3",
           "--scaled-mm-baseline", "--quant-ceiling", "--graph", "--accuracy"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["config"]["workload"] == "tiny_256x512x384"
    roof = d["roofline"]
    assert roof["bound"] == "mfma" and roof["peak"] == 5000.0 and 0 < roof["frac"] < 1
    assert roof["algorithmic_flops_per_launch"] == 2 * 256 * 384 * 512
    if d["clock"] and d["clock"].get("gfx_mhz_median"):
        adj = roof["clock_adjusted"]
        assert adj["peak"] == pytest.approx(5000.0 * d["clock"]["gfx_mhz_median"] / 2400.0, rel=1e-3)
        assert adj["frac"] == pytest.approx(roof["achieved"] / adj["peak"], abs=1e-4)
    q = d["quant_roofline"]
    assert q["bound"] == "hbm" and 0 < q["frac"] < 1
    calls = {c["call"] for c in q["cold_per_call"]}
    assert calls == {"weights", "tiny.x act"}
    for c in q["cold_per_call"]:
        assert c["copy_same_input_us"] > 0 and c["copy_time_over_quant_time"] > 0
    (g,) = d["per_gemm"]
    assert g["gemm"] == "tiny.fprop" and g["incl_quant_tflops"] < g["gemm_tflops"]
    smm = d["scaled_mm_baseline"]["per_gemm"]
    assert [x["gemm"] for x in smm] == ["tiny.fprop"] and smm[0]["hipblaslt_tensorwise_us"] > 0
    assert d["graph_replay"]["ms_per_step"] > 0
    assert d["cpu_baseline"]["kind"] == "oracle" and d["cpu_baseline"]["value"] > 0
    assert d["cpu_baseline"]["host"]["os_cpu_count"] >= 1
    assert d["bf16_baseline"]["value"] > 0
    acc = d["accuracy"]
    (p,) = acc["per_gemm"]
    assert p["gemm"] == "tiny.fprop" and set(p) == {"gemm", "fp32", "bf16"}
    # E4M3 keeps 3 mantissa bits: a few per cent normwise; bf16 inputs are exact
    assert 1e-3 < p["fp32"]["normwise"] < 0.1 and p["bf16"]["normwise"] < 1e-2
