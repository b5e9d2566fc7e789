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


def test_pmc_summary_derives_busy_clock_and_calibrated_bytes(tmp_path, monkeypatch):
    """Two counter runs of the same program (one per directory): the MFMA
    busy fraction is busy cycles over 1024 SIMDs x (GRBM cycles / 8 XCDs),
    and HBM bytes are the KiB counters scaled by the 1 GiB copy's reading."""
    hdr = ('"Correlation_Id","Dispatch_Id","Agent_Id","Queue_Id","Process_Id","Thread_Id",'
           '"Grid_Size","Kernel_Id","Kernel_Name","Workgroup_Size","LDS_Block_Size",'
           '"Scratch_Size","VGPR_Count","Accum_VGPR_Count","SGPR_Count","Counter_Name",'
           '"Counter_Value","Start_Timestamp","End_Timestamp"\n')

    def row(d, name, c, v, t0, t1):
        return f'{d},{d},"Agent 1",1,1,1,256,1,"{name}",256,0,0,8,0,16,"{c}",{v},{t0},{t1}\n'

    g = "void ns::(anonymous namespace)::gemm_kernel<false, false, 3, 1>(unsigned char const*)"
    cp = "void at::native::elementwise_kernel<copy_functor>(int)"
    a = tmp_path / "a" / "x"
    a.mkdir(parents=True)
    # 100 us at 2 GHz: GRBM counts 8 x 200000 cycles; MFMA busy 40 % of 1024 SIMDs
    (a / "p_counter_collection.csv").write_text(
        hdr + row(1, g, "GRBM_GUI_ACTIVE", 1600000, 0, 100000)
        + row(1, g, "SQ_VALU_MFMA_BUSY_CYCLES", 0.4 * 1024 * 200000, 0, 100000))
    b = tmp_path / "b"
    b.mkdir()
    # the copy reads half of what moved (factor 2); the GEMM fetches 100 MiB as counted
    (b / "q_counter_collection.csv").write_text(
        hdr + row(1, cp, "FETCH_SIZE", 512 * 1024, 0, 10) + row(2, g, "FETCH_SIZE", 100 * 1024, 0, 100000))
    c = tmp_path / "c"
    c.mkdir()
    (c / "q_counter_collection.csv").write_text(
        hdr + row(1, cp, "WRITE_SIZE", 1024 * 1024, 0, 10) + row(2, g, "WRITE_SIZE", 50 * 1024, 0, 100000))
    out_json = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out_json))
    md = bench.summarize_pmc([str(tmp_path / "a"), str(b), str(c)], write_traffic=True)
    line = [x for x in md.splitlines() if "gemm_kernel<false, false, 3, 1>" in x][0]
    assert "| 2.00 |" in line and "| 40.0% |" in line
    rec = json.loads(out_json.read_text())
    assert rec["fetch_factor"] == 2.0 and rec["write_factor"] == 1.0
    assert rec["hbm_bytes_per_launch"] == int((200 + 50) * 1024 * 1024)
    assert rec["gemm_source_sha256_16"] == bench.gemm_source_hash()


def test_rel_errors_normwise_and_worst_element():
    import numpy as np

    R = np.array([[3.0, 4.0], [0.0, 0.0]])
    assert bench.rel_errors(R, R) == {"normwise": 0.0, "max_over_rms": 0.0}
    C = R.copy()
    C[1, 1] = 0.5  # ||R||_F = 5, rms = 2.5
    e = bench.rel_errors(C, R)
    assert e["normwise"] == 0.1 and e["max_over_rms"] == 0.2
    assert bench.rel_errors(C.astype(np.float32), R)["normwise"] == 0.1


def test_trace_summary_counts_a_two_launch_gemm_call_once(tmp_path):
    """--summarize-trace: a pass of the tiny workload (one GEMM) whose call
    is two gemm kernel launches and a split-K reduction (the power-of-two
    kernel's whole-wave plan) gives one call whose time is all three."""
    import sqlite3

    db = tmp_path / "t.db"
    con = sqlite3.connect(db)
    con.execute("create table kernels (name text, start integer, duration integer)")
    t = 0
    # 1 warm-up + 2 headline + 2 instrumented passes of 4 dispatches each
    for _ in range(5):
        for name, d in (("quantize_dual_ct_kernel<0, 128, true, true>", 5000),
                        ("gemm_mx4_kernel<false, false, 3, 3>", 100000),
                        ("gemm_mx4_kernel<false, false, 3, 3>", 40000),
                        ("splitk_reduce_kernel<2>", 10000)):
            con.execute("insert into kernels values (?, ?, ?)", (name, t, d))
            t += d
    con.commit()
    con.close()
    md = bench.summarize_trace(str(db), 1, 2, "tiny_256x512x384")
    line = [x for x in md.splitlines() if x.startswith("GEMM calls per pass")][0]
    assert "GEMM calls per pass: 1 (2 gemm kernel launches)" in line, line
    assert "150.00 us" in line and "140.00 us per call" in line, line
