"""Opt-in input check: with BFP8_DEBUG set, every quantiser scans its input
and returns BFP8_ERR_NONFINITE (launching nothing) on Inf or NaN; without it,
the same calls succeed.  The variable is read once per process, so each case
runs in a child process (one at a time) that reports what it saw."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import json, sys, torch
sys.path.insert(0, ROOT)
import blockwise_fp8_gemm_bfp8_amd as bfp8
res = {}
def code(fn):
    try:
        fn()
        torch.cuda.synchronize()
        return 0
    except bfp8.BFP8Error as e:
        return e.code
for dt in (torch.bfloat16, torch.float32):
    name = str(dt).split(".")[-1]
    good = torch.randn(256, 256, generator=torch.Generator().manual_seed(0)).to(dt).cuda()
    for bad_val in ("nan", "inf", "-inf"):
        x = good.clone()
        x[131, 77] = float(bad_val)
        key = f"{name}.{bad_val}"
        res[key + ".act"] = code(lambda: bfp8.quantize_act(x))
        res[key + ".transposed"] = code(lambda: bfp8.quantize_act_transposed(x))
        res[key + ".dual"] = code(lambda: bfp8.quantize_act_dual(x))
        res[key + ".weight"] = code(lambda: bfp8.quantize_weight(x))
        res[key + ".batch"] = code(lambda: bfp8.quantize_weight_batch([good, x]))
        res[key + ".mx_dual"] = code(lambda: bfp8.quantize_mx_act_dual(x, 32))
        res[key + ".mx_weight"] = code(lambda: bfp8.quantize_mx_weight(x))
    q1, s1 = bfp8.quantize_act(good)
    res[name + ".finite.act"] = code(lambda: bfp8.quantize_act(good))
    res[name + ".finite.codes"] = [int(v) for v in q1[:4, :8].flatten().tolist()]
print("RESULT " + json.dumps(res), flush=True)
"""


def run_child(debug):
    env = dict(os.environ)
    if debug:
        env["BFP8_DEBUG"] = "1"
    else:
        env.pop("BFP8_DEBUG", None)
    out = subprocess.run([sys.executable, "-c", CHILD.replace("ROOT", repr(ROOT))], env=env,
                         capture_output=True, text=True, timeout=240)
    assert out.returncode == 0, out.stderr[-2000:]
    line = [l for l in out.stdout.splitlines() if l.startswith("RESULT ")][-1]
    return json.loads(line[len("RESULT "):])


def test_debug_mode_reports_nonfinite_inputs():
    on = run_child(True)
    off = run_child(False)
    for key, v in on.items():
        if ".finite." in key:
            continue
        assert v == 9, (key, v)          # BFP8_ERR_NONFINITE
        assert off[key] == 0, (key, off[key])
    for dt in ("bfloat16", "float32"):
        assert on[dt + ".finite.act"] == 0
        assert on[dt + ".finite.codes"] == off[dt + ".finite.codes"]
