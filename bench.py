"""Benchmark: blockwise-FP8 linear layers (quantise + GEMM) on one MI355X.

A step is one full pass of the hot path over one batch of synthetic input.
The default workload is one Puro-2B decoder layer's four linears at M = 16384
tokens (QKV 2048->4096, o_proj 2048->2048, gate/up 2048->12288, down
6144->2048): weight quantisation, activation quantisation and the fprop GEMM;
gradient quantisation and the dgrad GEMM; token-axis quantisation of dY and X
and the wgrad GEMM -- 12 GEMMs, 4.95 TFLOP.  Inputs are resident in HBM before
any timed region.  Prints ONE JSON line on stdout; details go to stderr.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--scales fp32|mx128|mx32] [--reps R] [--no-sweep]
                  [--no-cpu-baseline] [--no-bf16-baseline] [--copy-calibration]
                  [--scaled-mm-baseline] [--quant-ceiling] [--graph]
                  [--summarize-trace DB | --summarize-pmc DIR... [--write-traffic]]

Phases, in order (each after a synchronisation):
  1. W warm-up passes;
  2. the headline: exactly K passes bracketed by synchronisations; `value` is
     the workload's flops per pass over the mean pass time.  Each pass is also
     bracketed by a pair of HIP events (fence-free, on the launch stream), which
     give the median and p10/p90 of the pass time;
  2b. with --graph: the pass captured once into a HIP graph (no memset, no
     allocation in it) and K replays timed the same way (`graph_replay`);
  3. an instrumented copy of the same K passes, every kernel call bracketed
     by its own pair of events: each call's median launch time over the K
     passes, from which `roofline` (the GEMM family: mean flops per launch
     over mean launch time) and `quant_roofline` (the quantisers: bytes) are
     computed;
  4. a per-call sweep (unless --no-sweep): every kernel call of the pass run R
     times (default 50), each repetition after a read of a 1 GiB buffer that
     flushes the L2 caches and the 256 MB last-level cache, giving cold
     median / p10 / p90 per call, the per-GEMM TFLOP/s including the share of
     quantisation that feeds it, 2MNK / (t_act_quant + t_gemm), and the weight
     quantisation time amortised over the 64 micro-batches of one optimizer step.
  5. a clock window: passes back to back for about 2 s while amd-smi samples
     the graphics clock and the socket power (`clock`), with the sustained
     throughput of that window.

--scales picks the scale format of the pass: fp32 (float32 amax/448 scales,
promotion on the VALU; the default and the headline), mx128 (the same groups
with power-of-two E8M0 scales applied by the scaled MFMA) or mx32 (MXFP8, 1x32
power-of-two groups).  The line also carries `bf16_baseline`: the same GEMMs on
the unquantised bf16 tensors through torch.matmul (hipBLASLt), timed the same
way, for the FP8-over-BF16 ratio.
"""

import argparse
import hashlib
import json
import os
import platform
import statistics
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "blockwise-FP8 GEMM TFLOP/s incl. quantize at Puro-2B shapes; % FP8 MFMA peak"
FP8_DENSE_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 MFMA, published
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
PEAK_GFX_MHZ = 2400.0           # the engine clock the FP8 peak is quoted at
MICROBATCHES_PER_STEP = 64      # 1536 sequences / (12 data-parallel ranks x 2 per micro-batch)
DEFAULT_WORKLOAD = "layer_fwd_bwd_m16384"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_traffic.json")
GEMM_SOURCE = os.path.join(ROOT, "blockwise_fp8_gemm_bfp8_amd", "csrc", "gemm.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def pct(xs, q):
    """q-th percentile (0..100) by linear interpolation."""
    xs = sorted(xs)
    if not xs:
        return None
    k = (len(xs) - 1) * q / 100.0
    lo, hi = int(k), min(int(k) + 1, len(xs) - 1)
    return xs[lo] + (xs[hi] - xs[lo]) * (k - lo)


def gemm_source_hash():
    with open(GEMM_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic():
    """HBM bytes per GEMM launch from the committed rocprofv3 --pmc summary,
    only if it was measured on the current GEMM source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("gemm_source_sha256_16") != gemm_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


class ClockSampler:
    """amd-smi in a background thread: graphics clock (mean over the XCDs) and
    socket power, sampled back to back while the GPU work runs."""

    def __init__(self):
        self.samples = []
        self._stop = threading.Event()
        self._t = None

    def _one(self):
        out = subprocess.run(["amd-smi", "metric", "-c", "-p", "--json"], capture_output=True,
                             text=True, timeout=20)
        data = json.loads(out.stdout)
        gpus = data if isinstance(data, list) else data.get("gpu_data", [data])
        g = gpus[0]
        clocks = []
        for k, v in g.get("clock", {}).items():
            if k.startswith("gfx") and isinstance(v, dict):
                c = v.get("clk", {})
                c = c.get("value") if isinstance(c, dict) else c
                if isinstance(c, (int, float)):
                    clocks.append(float(c))
        p = g.get("power", {}).get("socket_power", {})
        p = p.get("value") if isinstance(p, dict) else p
        if clocks:
            self.samples.append((time.perf_counter(), sum(clocks) / len(clocks),
                                 float(p) if isinstance(p, (int, float)) else None))

    def _loop(self):
        while not self._stop.is_set():
            try:
                self._one()
            except Exception:  # amd-smi missing or its output not understood
                return

    def start(self):
        self._t = threading.Thread(target=self._loop, daemon=True)
        self._t.start()

    def stop(self):
        self._stop.set()
        if self._t is not None:
            self._t.join(timeout=30)

    def summary(self, t0, t1):
        s = [x for x in self.samples if t0 <= x[0] <= t1]
        if not s:
            return None
        clk = [x[1] for x in s]
        pw = [x[2] for x in s if x[2] is not None]
        return {"gfx_mhz_median": round(statistics.median(clk), 1), "gfx_mhz_min": min(clk),
                "gfx_mhz_max": max(clk), "socket_power_w_median":
                round(statistics.median(pw), 1) if pw else None, "samples": len(s),
                "source": "amd-smi metric -c -p, mean over the 8 XCD clocks"}


def host_facts(threads):
    model = platform.processor() or None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "blas_threads": threads}


def cpu_baseline(workload_name, tokens_sample, scales="fp32"):
    """The oracle (numpy, float64 GEMM) on the same workload with M cut to
    `tokens_sample` tokens: every quantiser and all GEMMs of the step."""
    import numpy as np  # noqa: F401

    import oracle
    from workloads import WORKLOADS, make_inputs, to_numpy_input

    try:
        from threadpoolctl import threadpool_info

        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    wl = WORKLOADS[workload_name]
    t = make_inputs(workload_name)
    M = min(tokens_sample, wl.tokens)
    flops = 0
    t0 = time.perf_counter()
    if scales != "fp32":
        grp = 32 if scales == "mx32" else 128
        mode = "mx32" if grp == 32 else "act"
        for L in wl.linears:
            x = to_numpy_input(t["x." + L.name])[:M]
            w = to_numpy_input(t["w." + L.name])
            dy = to_numpy_input(t["dy." + L.name])[:M]
            xq, xs = oracle.quantize_mx_act(x, grp)
            dq, ds = oracle.quantize_mx_act(dy, grp)
            if grp == 32:
                wq, ws = oracle.quantize_mx_act(w, 32)
                wqt, wst = oracle.quantize_mx_act_transposed(w, 32)
                oracle.gemm_mx_ref("NT", xq, xs, mode, wq, ws, mode)
                oracle.gemm_mx_ref("NT", dq, ds, mode, wqt, wst, mode)
            else:
                wq, ws = oracle.quantize_mx_weight(w)
                oracle.gemm_mx_ref("NT", xq, xs, mode, wq, ws, "block")
                oracle.gemm_mx_ref("NN", dq, ds, mode, wq, ws, "block")
            aq, as_ = oracle.quantize_mx_act_transposed(dy, grp)
            bq, bs = oracle.quantize_mx_act_transposed(x, grp)
            oracle.gemm_mx_ref("NT", aq, as_, mode, bq, bs, mode)
            flops += 3 * 2 * M * L.out_features * L.in_features
    for L in (wl.linears if scales == "fp32" else []):
        x = to_numpy_input(t["x." + L.name])[:M]
        w = to_numpy_input(t["w." + L.name])
        wq, ws = oracle.quantize_weight(w)
        if "fprop" in wl.roles:
            xq, xs = oracle.quantize_act(x)
            oracle.gemm_ref("NT", xq, xs, "act", wq, ws, "block")
            flops += 2 * M * L.out_features * L.in_features
        if "dgrad" in wl.roles or "wgrad" in wl.roles:
            dy = to_numpy_input(t["dy." + L.name])[:M]
        if "dgrad" in wl.roles:
            dq, ds = oracle.quantize_act(dy)
            oracle.gemm_ref("NN", dq, ds, "act", wq, ws, "block")
            flops += 2 * M * L.out_features * L.in_features
        if "wgrad" in wl.roles:
            aq, as_ = oracle.quantize_act_transposed(dy)
            bq, bs = oracle.quantize_act_transposed(x)
            oracle.gemm_ref("NT", aq, as_, "act", bq, bs, "act")
            flops += 2 * M * L.out_features * L.in_features
    dt = time.perf_counter() - t0
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{workload_name} with M cut to {M} tokens (all quantisers and GEMMs of "
                  f"one step, {scales} scales, {flops / 1e9:.1f} GFLOP, {dt:.1f} s)",
        "host": host_facts(int(threads)),
    }


def bf16_baseline(tensors, wl, steps, fp8_value):
    """The step's GEMMs on the unquantised bf16 tensors via torch.matmul
    (hipBLASLt), no quantisation: fprop X W^T, dgrad dY W, wgrad dY^T X."""
    import torch

    # every operand contiguous: the transposes W^T and dY^T are materialised
    # once, outside the timed steps, so each product is a plain row-major
    # 2-D matmul
    lin = [(tensors["x." + L.name], tensors["w." + L.name], tensors.get("dy." + L.name),
            tensors["w." + L.name].t().contiguous(),
            tensors["dy." + L.name].t().contiguous() if "dy." + L.name in tensors else None)
           for L in wl.linears]

    def step():
        if "fprop" in wl.roles:
            for x, _, _, wt, _ in lin:
                torch.matmul(x, wt)
        for x, w, dy, _, dyt in lin:
            if "dgrad" in wl.roles:
                torch.matmul(dy, w)
            if "wgrad" in wl.roles:
                torch.matmul(dyt, x)

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    value = wl.flops / dt / 1e12
    log(f"[bench] bf16 baseline (torch.matmul): {dt * 1e3:.3f} ms per step, {value:.1f} TFLOP/s")
    return {"value": round(value, 2), "unit": "TFLOP/s", "ms_per_step": round(dt * 1e3, 4),
            "kind": "the same GEMMs in bf16 via torch.matmul (hipBLASLt), unquantised",
            "fp8_over_bf16": round(fp8_value / value, 3)}


def rel_errors(C, R):
    """Errors of C against the reference R (float64 arrays of one shape):
    normwise ||C - R||_F / ||R||_F, and the largest |C - R| over rms(R)."""
    import numpy as np

    d = np.asarray(C, np.float64) - np.asarray(R, np.float64)
    rn = float(np.linalg.norm(R))
    rms = rn / (R.size ** 0.5) if R.size else 0.0
    return {"normwise": round(float(np.linalg.norm(d)) / rn, 6) if rn > 0 else 0.0,
            "max_over_rms": round(float(np.abs(d).max()) / rms, 5) if rms > 0 else 0.0}


def accuracy_report(tensors, wl, hp_main, rows=128, seed=0):
    """Accuracy of the scale formats (the f2 / f4 comparison): every GEMM of
    one pass, run with float32 scales (1x128 / 128x128 groups), power-of-two
    scales on the same groups (mx128) and 1x32 power-of-two groups (mx32),
    and the same product in bf16 through hipBLASLt, each against the float64
    product of the unquantised inputs, on `rows` sampled output rows (tokens
    for fprop and dgrad, output features for wgrad)."""
    import numpy as np
    import torch

    from blockwise_fp8_gemm_bfp8_amd.hotpath import HotPath

    g = np.random.default_rng(seed)
    names = [L.name for L in wl.linears]
    f64 = lambda t: t.double().cpu().numpy()
    pick = {}
    ref = {}
    for L in wl.linears:
        x, w, dy = tensors["x." + L.name], tensors["w." + L.name], tensors.get("dy." + L.name)
        M = x.shape[0]
        tr = np.sort(g.choice(M, min(rows, M), replace=False))
        fr = np.sort(g.choice(w.shape[0], min(rows, w.shape[0]), replace=False))
        pick[L.name] = (tr, fr)
        ti = torch.from_numpy(tr).to(x.device)
        fi = torch.from_numpy(fr).to(x.device)
        wd = f64(w)
        if "fprop" in wl.roles:
            ref[(L.name, "fprop")] = f64(x.index_select(0, ti)) @ wd.T
        if dy is not None and "dgrad" in wl.roles:
            ref[(L.name, "dgrad")] = f64(dy.index_select(0, ti)) @ wd
        if dy is not None and "wgrad" in wl.roles:
            ref[(L.name, "wgrad")] = f64(dy.index_select(1, fi)).T @ f64(x)
    key = {"fprop": "y", "dgrad": "dx", "wgrad": "dw"}
    out = {k: {} for k in ref}
    formats = ["fp32", "mx128", "mx32"] if set(wl.roles) == {"fprop", "dgrad", "wgrad"} else ["fp32"]
    for sc in formats:
        hp = hp_main if hp_main.scales == sc else HotPath(tensors, names, wl.roles, scales=sc)
        hp.run()
        torch.cuda.synchronize()
        for L in hp.layers:
            tr, fr = pick[L.name]
            for role in ("fprop", "dgrad", "wgrad"):
                if (L.name, role) not in ref:
                    continue
                idx = torch.from_numpy(fr if role == "wgrad" else tr).to(L.x.device)
                got = f64(L.buf[key[role]].index_select(0, idx))
                out[(L.name, role)][sc] = rel_errors(got, ref[(L.name, role)])
        if hp is not hp_main:
            del hp
            torch.cuda.empty_cache()
    # the same products in bf16 (contiguous 2-D operands only)
    for L in wl.linears:
        x, w, dy = tensors["x." + L.name], tensors["w." + L.name], tensors.get("dy." + L.name)
        tr, fr = pick[L.name]
        ti = torch.from_numpy(tr).to(x.device)
        fi = torch.from_numpy(fr).to(x.device)
        xb, wb = x.to(torch.bfloat16), w.to(torch.bfloat16)
        prods = {}
        if (L.name, "fprop") in ref:
            prods["fprop"] = torch.matmul(xb.index_select(0, ti), wb.t().contiguous())
        if (L.name, "dgrad") in ref:
            prods["dgrad"] = torch.matmul(dy.to(torch.bfloat16).index_select(0, ti), wb)
        if (L.name, "wgrad") in ref:
            prods["wgrad"] = torch.matmul(dy.to(torch.bfloat16).index_select(1, fi).t().contiguous(), xb)
        for role, c in prods.items():
            out[(L.name, role)]["bf16"] = rel_errors(f64(c), ref[(L.name, role)])
    per = [{"gemm": f"{n}.{r}", **v} for (n, r), v in out.items()]
    summary = {}
    for f in formats + ["bf16"]:
        vals = [p[f]["normwise"] for p in per if f in p]
        if vals:
            summary[f] = {"normwise_mean": round(sum(vals) / len(vals), 6),
                          "normwise_max": round(max(vals), 6)}
    for p in per:
        log(f"[bench] accuracy {p['gemm']:15s} " + "  ".join(
            f"{f} {p[f]['normwise']:.2e}" for f in formats + ["bf16"] if f in p))
    return {"reference": "float64 product of the unquantised inputs (the workload's bf16 / fp32 "
                         "tensors), sampled output rows", "rows_sampled": rows,
            "metric": "normwise = ||C - R||_F / ||R||_F; max_over_rms = max |C - R| / rms(R)",
            "formats": {"fp32": "float32 scales amax/448, 1x128 act / 128x128 weight groups",
                        "mx128": "power-of-two (E8M0) scales on the same groups",
                        "mx32": "MXFP8: 1x32 power-of-two groups on every operand",
                        "bf16": "unquantised bf16 operands, hipBLASLt"},
            "summary": summary, "per_gemm": per}


def family_roofline(hp, mean_us, kind, fields):
    """Roofline of one kernel family from the instrumented passes: the mean
    algorithmic work per launch over the mean launch time (each call's time
    being its median over the passes)."""
    idx = [i for i, op in enumerate(hp.ops) if op.kind in kind]
    if not idx:
        return None
    t = sum(mean_us[i] for i in idx) / len(idx)
    if fields == "flops":
        work = sum(hp.ops[i].flops for i in idx) / len(idx)
        ach = work / (t * 1e-6) / 1e12
        return {"bound": "mfma", "achieved": round(ach, 1), "peak": FP8_DENSE_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / FP8_DENSE_PEAK_TFLOPS, 4),
                "avg_launch_us": round(t, 2), "launches_per_step": len(idx),
                "algorithmic_flops_per_launch": int(work)}
    work = sum(hp.ops[i].bytes for i in idx) / len(idx)
    ach = work / (t * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "avg_launch_us": round(t, 2),
            "launches_per_step": len(idx), "algorithmic_bytes_per_launch": int(work)}


def sweep(hp, reps):
    """Every kernel call of the pass, `reps` times, each after a read of a
    1 GiB buffer that evicts the L2 caches and the 256 MB last-level cache
    (a read, so no dirty lines are left for the timed call to write back):
    cold median / p10 / p90 in microseconds."""
    import torch

    from blockwise_fp8_gemm_bfp8_amd.hotpath import TimingEvent

    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    out = []
    for op in hp.ops:
        evs = []
        for _ in range(reps):
            torch.sum(flush, dim=(0,), out=sink)
            s, e = TimingEvent(), TimingEvent()
            s.record()
            op.fn()
            e.record()
            evs.append((s, e))
        torch.cuda.synchronize()
        us = [s.elapsed_time(e) * 1e3 for s, e in evs]
        out.append({"median": statistics.median(us), "p10": pct(us, 10), "p90": pct(us, 90)})
    del flush
    return out


def scaled_mm_baseline(hp, reps):
    """hipBLASLt's per-tensor-scaled FP8 GEMM (torch._scaled_mm, unit scales,
    bf16 output) on each GEMM's own E4M3 code operands, beside the same call
    of this library, both timed cold as in the sweep (median of `reps`).  The
    vendor kernel applies no per-block scales and no promotion: it is the
    matrix-core rate of a tuned kernel on the same bytes."""
    import torch

    from blockwise_fp8_gemm_bfp8_amd.hotpath import TimingEvent

    f8 = torch.float8_e4m3fn
    one = torch.ones((), dtype=torch.float32, device="cuda")
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")

    def cold(fn):
        evs = []
        for _ in range(reps):
            torch.sum(flush, dim=(0,), out=sink)
            s, e = TimingEvent(), TimingEvent()
            s.record()
            fn()
            e.record()
            evs.append((s, e))
        torch.cuda.synchronize()
        return statistics.median([s.elapsed_time(e) * 1e3 for s, e in evs])

    out = []
    for op in hp.ops:
        if op.kind != "gemm" or op.codes is None:
            continue
        a, b = op.codes
        if op.layout == "NT":      # A [M][K], B [N][K]
            A, Bt = a.view(f8), b.view(f8)
        elif op.layout == "NN":    # A [M][K], B [K][N]: B^T materialised once
            A, Bt = a.view(f8), b.t().contiguous().view(f8)
        else:
            continue

        def vendor(A=A, Bt=Bt):
            torch._scaled_mm(A, Bt.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)

        vendor()
        op.fn()
        torch.cuda.synchronize()
        tv, to = cold(vendor), cold(op.fn)
        M, N, K = op.mnk
        rec = {"gemm": op.label, "layout": op.layout, "mnk": [M, N, K],
               "hipblaslt_tensorwise_us": round(tv, 2), "ours_us": round(to, 2),
               "hipblaslt_tflops": round(op.flops / (tv * 1e-6) / 1e12, 1),
               "ours_tflops": round(op.flops / (to * 1e-6) / 1e12, 1)}
        out.append(rec)
        log(f"[bench] vs hipBLASLt {op.label:15s} {rec['hipblaslt_tensorwise_us']:8.1f} us "
            f"({rec['hipblaslt_tflops']:6.1f} TFLOP/s)   ours {rec['ours_us']:8.1f} us "
            f"({rec['ours_tflops']:6.1f})")
    del flush
    tv = sum(r["hipblaslt_tensorwise_us"] for r in out)
    to = sum(r["ours_us"] for r in out)
    fl = sum(op.flops for op in hp.ops if op.kind == "gemm" and op.codes is not None
             and op.layout in ("NT", "NN"))
    return {"kind": "torch._scaled_mm (hipBLASLt), per-tensor unit scales, on the pass's own "
                    "E4M3 codes; cold median per GEMM",
            "hipblaslt_tflops": round(fl / (tv * 1e-6) / 1e12, 1) if tv else None,
            "ours_tflops": round(fl / (to * 1e-6) / 1e12, 1) if to else None,
            "per_gemm": out}


def copy_ceiling(hp, reps):
    """For each quantiser call: a plain device copy (torch copy_) of a
    contiguous buffer with as many elements, of the same dtype, as the call
    reads, timed cold like the sweep.  The copy reads and writes every
    byte once with no arithmetic and one launch: the access-volume ceiling
    for a kernel of that size (it moves at least the quantiser's bytes --
    exactly them for the dual quantiser, whose two E4M3 outputs equal the
    bf16 input in size).  Returns {op index: (median us, bytes moved)}."""
    import torch

    from blockwise_fp8_gemm_bfp8_amd.hotpath import TimingEvent

    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    out = {}
    for i, op in enumerate(hp.ops):
        if op.kind == "gemm" or not op.src:
            continue
        n = sum(t.numel() for t in op.src)
        a = torch.ones(n, dtype=op.src[0].dtype, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        evs = []
        for _ in range(reps):
            torch.sum(flush, dim=(0,), out=sink)
            s, e = TimingEvent(), TimingEvent()
            s.record()
            b.copy_(a)
            e.record()
            evs.append((s, e))
        torch.cuda.synchronize()
        out[i] = (statistics.median([s.elapsed_time(e) * 1e3 for s, e in evs]),
                  2 * n * a.element_size())
        del a, b
    del flush
    return out


XCDS = 8            # MI355X: GRBM_GUI_ACTIVE counts once per XCD
SIMDS = 256 * 4     # 256 CUs x 4 SIMDs


def summarize_pmc(dirs, write_traffic=False, workload=DEFAULT_WORKLOAD):
    """Markdown summary of rocprofv3 --pmc runs of this script (the
    *counter_collection.csv files under each directory), per kernel: mean
    duration, and whichever of these the counters allow -- graphics clock
    (GRBM_GUI_ACTIVE over the 8 XCDs), MFMA busy fraction
    (SQ_VALU_MFMA_BUSY_CYCLES over 1024 SIMDs), FP8 rate from the MFMA op
    count, LDS issue stalls, bank conflicts and unaligned stalls, and HBM
    bytes from FETCH_SIZE / WRITE_SIZE (KiB) scaled by what the same counter
    reads for the 1 GiB copy of --copy-calibration.  With write_traffic, the
    mean GEMM-kernel bytes per launch go to profiles/gemm_traffic.json,
    stamped with the GEMM source hash."""
    import csv
    import glob

    per = {}
    copy = {}
    for d in dirs:
        for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            disp = {}
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    e = disp.setdefault(r["Dispatch_Id"], [r["Kernel_Name"], int(r["End_Timestamp"])
                                                           - int(r["Start_Timestamp"]), {}])
                    e[2][r["Counter_Name"]] = float(r["Counter_Value"])
            for name, dur, cs in disp.values():
                if "copy" in name.lower():
                    for c in ("FETCH_SIZE", "WRITE_SIZE"):
                        if c in cs:
                            copy[c] = max(copy.get(c, 0.0), cs[c])
                    continue
                k = per.setdefault(_short_kernel_name(name), {"_dur": [], "_n": {}})
                k["_dur"].append(dur)
                for c, v in cs.items():
                    k.setdefault(c, []).append(v)
                k["_n"][f] = k["_n"].get(f, 0) + 1
    gib_kib = float(1 << 20)
    factor = {c: gib_kib / copy[c] for c in copy if copy[c] > 0}

    def m(k, c):
        v = k.get(c)
        return sum(v) / len(v) if v else None

    rows = []
    traffic = []
    for name, k in sorted(per.items(), key=lambda kv: -sum(kv[1]["_dur"])):
        dur = sum(k["_dur"]) / len(k["_dur"])  # ns
        launches = max(k["_n"].values())
        r = {"kernel": name, "launches": launches, "us": dur / 1e3}
        g = m(k, "GRBM_GUI_ACTIVE")
        if g:
            r["ghz"] = g / XCDS / dur
            b = m(k, "SQ_VALU_MFMA_BUSY_CYCLES")
            if b is not None:
                r["mfma_busy"] = b / (SIMDS * g / XCDS)
        mops = m(k, "SQ_INSTS_VALU_MFMA_MOPS_F8")
        if mops:
            r["fp8_tflops"] = mops * 512 / (dur * 1e-9) / 1e12
        wc = m(k, "SQ_WAVE_CYCLES")
        if wc:
            for c, key in (("SQ_WAIT_INST_LDS", "wait_lds_issue"), ("SQ_WAIT_ANY", "wait_any")):
                if m(k, c) is not None:
                    r[key] = m(k, c) / wc
        act = m(k, "SQ_LDS_IDX_ACTIVE")
        if act:
            if m(k, "SQ_LDS_BANK_CONFLICT") is not None:
                r["lds_bank_conflict"] = m(k, "SQ_LDS_BANK_CONFLICT") / act
            if m(k, "SQ_LDS_UNALIGNED_STALL") is not None:
                r["lds_unaligned"] = m(k, "SQ_LDS_UNALIGNED_STALL") / act
        nbytes = 0.0
        for c, key in (("FETCH_SIZE", "fetch_mb"), ("WRITE_SIZE", "write_mb")):
            if m(k, c) is not None and c in factor:
                r[key] = m(k, c) * 1024 * factor[c] / 1e6
                nbytes += r[key] * 1e6
        if "fetch_mb" in r and "write_mb" in r:
            r["hbm_gbs"] = nbytes / (dur * 1e-9) / 1e9
            if name.startswith("gemm_kernel") or name.startswith("gemm_mx4_kernel"):
                traffic += [nbytes] * launches
        rows.append(r)
    cols = [("launches", "launches", "{:d}"), ("us", "mean us", "{:.1f}"), ("ghz", "GHz", "{:.2f}"),
            ("mfma_busy", "MFMA busy", "{:.1%}"), ("fp8_tflops", "FP8 TFLOP/s", "{:.0f}"),
            ("wait_lds_issue", "LDS issue wait", "{:.1%}"), ("wait_any", "waitcnt/barrier", "{:.1%}"),
            ("lds_bank_conflict", "bank confl.", "{:.1%}"), ("lds_unaligned", "unaligned", "{:.1%}"),
            ("fetch_mb", "fetch MB", "{:.1f}"), ("write_mb", "write MB", "{:.1f}"),
            ("hbm_gbs", "HBM GB/s", "{:.0f}")]
    used = [c for c in cols if any(c[0] in r for r in rows)]
    out = ["| kernel | " + " | ".join(c[1] for c in used) + " |",
           "|---|" + "---|" * len(used)]
    for r in rows:
        out.append(f"| `{r['kernel']}` | " + " | ".join(
            (c[2].format(r[c[0]]) if c[0] in r else "") for c in used) + " |")
    if factor:
        out += ["", "Copy calibration (1 GiB torch copy): " + ", ".join(
            f"{c} reads {copy[c] / 1024:.1f} MiB -> factor {factor[c]:.3f}" for c in sorted(factor))]
    if traffic:
        mean = sum(traffic) / len(traffic)
        out += ["", f"GEMM kernels: {mean / 1e6:.1f} MB of HBM-side traffic per launch (mean over "
                    f"{len(traffic)} launches); GEMM source sha256[:16] = {gemm_source_hash()}."]
        if write_traffic:
            with open(TRAFFIC_FILE, "w") as fh:
                json.dump({"gemm_source_sha256_16": gemm_source_hash(),
                           "hbm_bytes_per_launch": int(mean),
                           "fetch_factor": factor.get("FETCH_SIZE"),
                           "write_factor": factor.get("WRITE_SIZE"), "workload": workload,
                           "summary": f"profiles/gemm_hbm_traffic_{workload}.md"}, fh, indent=1)
    return "\n".join(out)


def _short_kernel_name(name):
    """'void ns::(anonymous namespace)::gemm_kernel<false, true, 0, 1>(args)' ->
    'gemm_kernel<false, true, 0, 1>'."""
    import re

    m = re.search(r"(\w+)(<[^()]*>)?\(", name)
    return (m.group(1) + (m.group(2) or "")) if m else name[:80]


def summarize_trace(db, warmup, steps, workload=DEFAULT_WORKLOAD):
    """Markdown summary of a rocprofv3 --kernel-trace database of this
    script: every kernel over the whole run, then the timed passes alone.

    The first dispatches of the run are the W warm-up passes, then the K
    headline passes, then the K instrumented passes; a pass is found as the
    period of the dispatch sequence.  A GEMM call is its gemm kernel
    launches (two when the power-of-two kernel runs a split plan as whole
    tiles, then split tiles) plus the split-K reduction that follows, which
    is what the line's event timing brackets: the mean call is the pass's
    GEMM and reduction time over the workload's GEMM count."""
    import sqlite3

    con = sqlite3.connect(db)
    rows = con.execute("select name, duration from kernels order by start").fetchall()
    names = [_short_kernel_name(r[0]) for r in rows]
    dur = [r[1] / 1e3 for r in rows]  # us
    total = warmup + 2 * steps
    period = None
    for p in range(1, 400):
        if total * p <= len(names) and all(names[i] == names[i + p] for i in range((total - 1) * p)):
            period = p
            break
    lines = ["| kernel | calls | total us | avg us | % |", "|---|---|---|---|---|"]
    agg = {}
    for n, d in zip(names, dur):
        a = agg.setdefault(n, [0, 0.0])
        a[0] += 1
        a[1] += d
    grand = sum(a[1] for a in agg.values())
    for n, (c, t) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        lines.append(f"| `{n}` | {c} | {t:.1f} | {t / c:.2f} | {100 * t / grand:.1f} |")
    out = ["Every dispatch of the run:", ""] + lines
    if period is None:
        out += ["", "(no periodic pass structure found for the given --warmup / --steps)"]
        return "\n".join(out)
    a0, a1 = warmup * period, (warmup + steps) * period
    calls, kern = [], []
    per = {}
    for i in range(a0, a1):
        n = names[i]
        per.setdefault(n, []).append(dur[i])
        if n.startswith("gemm_kernel") or n.startswith("gemm_mx4_kernel"):
            calls.append(dur[i])
            kern.append(dur[i])
        elif n.startswith("splitk_reduce") and calls:
            calls[-1] += dur[i]
    out += ["", f"The {steps} headline passes alone (dispatches {a0}..{a1 - 1}, {period} per pass):",
            "", "| kernel | calls | avg us | median us |", "|---|---|---|---|"]
    for n, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"| `{n}` | {len(v)} | {sum(v) / len(v):.2f} | {statistics.median(v):.2f} |")
    if calls:
        from workloads import WORKLOADS

        n_calls = len(WORKLOADS[workload].gemms) * steps
        out += ["", f"GEMM calls per pass: {n_calls // steps} ({len(kern) // steps} gemm kernel "
                f"launches); mean GEMM call (its kernel launches + split-K reduction) "
                f"{sum(calls) / n_calls:.2f} us; gemm kernels alone {sum(kern) / n_calls:.2f} us "
                f"per call."]
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=1024)
    ap.add_argument("--scales", default="fp32", choices=["fp32", "mx128", "mx32"])
    ap.add_argument("--no-bf16-baseline", action="store_true")
    ap.add_argument("--reps", type=int, default=50, help="repetitions per call in the sweep")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--clock-window", type=float, default=2.0,
                    help="seconds of back-to-back passes sampled for the clock (0: none)")
    ap.add_argument("--summarize-trace", metavar="DB",
                    help="summarise a rocprofv3 kernel trace of this script (no GPU needed) "
                         "and exit; --steps / --warmup must match the traced run")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for HBM counter calibration)")
    ap.add_argument("--summarize-pmc", metavar="DIR", nargs="+",
                    help="summarise rocprofv3 --pmc runs of this script (no GPU needed) and exit")
    ap.add_argument("--write-traffic", action="store_true",
                    help="with --summarize-pmc: record the GEMM bytes per launch for the line")
    ap.add_argument("--scaled-mm-baseline", action="store_true",
                    help="also time hipBLASLt's per-tensor FP8 GEMM on the pass's own codes")
    ap.add_argument("--quant-ceiling", action="store_true",
                    help="with the sweep: time a plain copy of each quantiser's input volume")
    ap.add_argument("--accuracy", action="store_true",
                    help="also compare every GEMM in float32, mx128 and mx32 scales and in bf16 "
                         "against the float64 product of the unquantised inputs (sampled rows)")
    ap.add_argument("--graph", action="store_true",
                    help="also time K replays of the pass captured into one HIP graph")
    args = ap.parse_args()

    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.warmup, args.steps, args.workload))
        return
    if args.summarize_pmc:
        print(summarize_pmc(args.summarize_pmc, args.write_traffic, args.workload))
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library has no "
              "multi-GPU path -- each GPU runs the same data-parallel step independently.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from blockwise_fp8_gemm_bfp8_amd import build as _build

    if not os.path.exists(_build.LIB_PATH):
        _build.build()
    from blockwise_fp8_gemm_bfp8_amd.hotpath import HotPath, TimingEvent
    from workloads import WORKLOADS, make_inputs

    wl = WORKLOADS[args.workload]
    log(f"[bench] workload {wl.name}: generating inputs")
    tensors = {k: v.cuda() for k, v in make_inputs(wl.name).items()}
    if args.scales != "fp32" and set(wl.roles) != {"fprop", "dgrad", "wgrad"}:
        log("[bench] power-of-two scales run only on the full fprop + dgrad + wgrad layer")
        sys.exit(2)
    hp = HotPath(tensors, [L.name for L in wl.linears], wl.roles, scales=args.scales)
    flops_step = wl.flops

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        hp.run()
    torch.cuda.synchronize()

    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 1 GiB read + 1 GiB write")
        del a, b

    # ---- phase 2: the headline -------------------------------------------
    log(f"[bench] timing {args.steps} steps")
    step_ev = [(TimingEvent(), TimingEvent()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s, e in step_ev:
        s.record()
        hp.run()
        e.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed / args.steps * 1e3
    value = flops_step / (elapsed / args.steps) / 1e12
    step_ms = [s.elapsed_time(e) for s, e in step_ev]
    log(f"[bench] {ms_per_step:.3f} ms per step (wall), events median "
        f"{statistics.median(step_ms):.3f} ms, {value:.1f} TFLOP/s")

    # ---- phase 2b (--graph): the pass captured once, replayed K times --------
    graph = None
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            hp.run()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            hp.run()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        tg0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        gdt = (time.perf_counter() - tg0) / args.steps
        graph = {"ms_per_step": round(gdt * 1e3, 4),
                 "value": round(flops_step / gdt / 1e12, 2),
                 "kind": "the same pass captured once into a HIP graph, K replays timed the "
                         "same way (launch cost off the host)"}
        log(f"[bench] graph replay: {gdt * 1e3:.3f} ms per step, {graph['value']:.1f} TFLOP/s")
        del g

    # ---- phase 3: the same passes with every kernel call bracketed -----------
    # (every event is created before the passes are enqueued; per call, the
    # median over the K passes is the launch time used below -- a median, so
    # that one stalled launch does not move the roofline)
    pool = [(TimingEvent(), TimingEvent()) for _ in range(args.steps * len(hp.ops))]
    events = []
    torch.cuda.synchronize()
    k = 0
    for _ in range(args.steps):
        for i, op in enumerate(hp.ops):
            s, e = pool[k]
            k += 1
            s.record()
            op.fn()
            e.record()
            events.append((i, s, e))
    torch.cuda.synchronize()
    per_op = {}
    for i, s, e in events:
        per_op.setdefault(i, []).append(s.elapsed_time(e) * 1e3)
    mean_us = {i: statistics.median(v) for i, v in per_op.items()}
    spread = {i: (min(v), max(v)) for i, v in per_op.items()}
    roofline = family_roofline(hp, mean_us, ("gemm",), "flops")
    roofline["kernel"] = ("gemm_kernel: the blockwise FP8 GEMM launches of the step (float32 "
                          "scales; each call's time includes its split-K reduction kernel "
                          "where the call splits K)" if args.scales == "fp32" else
                          f"gemm_mx4_kernel ({args.scales}; each call's time includes its "
                          "split-K reduction kernel where the call splits K)")
    roofline["traffic"] = load_traffic() if args.scales == "fp32" else None
    qroof = family_roofline(hp, mean_us, ("quant", "weight_quant"), "bytes")
    if qroof is not None:
        qroof["kernel"] = ("the step's quantiser launches (activation, gradient and weight): "
                           "mean algorithmic bytes per launch over the mean launch time")
        qroof["per_call"] = [
            {"call": hp.ops[i].label, "us": round(mean_us[i], 2),
             "gbs": round(hp.ops[i].bytes / (mean_us[i] * 1e-6) / 1e9, 1),
             "frac": round(hp.ops[i].bytes / (mean_us[i] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
            for i in range(len(hp.ops)) if hp.ops[i].kind != "gemm"]

    # ---- phase 4: cold per-call sweep ----------------------------------------
    per_gemm = None
    weight_quant = None
    if not args.no_sweep:
        log(f"[bench] sweep: {args.reps} cold repetitions of each of {len(hp.ops)} calls")
        sw = sweep(hp, args.reps)
        act_us = {}
        for op, st in zip(hp.ops, sw):
            for g, share in op.feeds:
                act_us[g] = act_us.get(g, 0.0) + share * st["median"]
        per_gemm = []
        for op, st in zip(hp.ops, sw):
            if op.kind != "gemm":
                continue
            tq = act_us.get(op.label, 0.0)
            per_gemm.append({
                "gemm": op.label, "layout": op.layout, "mnk": list(op.mnk),
                "gemm_us": {k: round(v, 2) for k, v in st.items()},
                "gemm_tflops": round(op.flops / (st["median"] * 1e-6) / 1e12, 1),
                "act_quant_us": round(tq, 2),
                "incl_quant_tflops": round(op.flops / ((st["median"] + tq) * 1e-6) / 1e12, 1)})
            log(f"[bench] {op.label:15s} {op.layout} M,N,K={op.mnk}: median "
                f"{st['median']:8.1f} us (p10 {st['p10']:.1f}, p90 {st['p90']:.1f})  "
                f"{per_gemm[-1]['gemm_tflops']:7.1f} TFLOP/s; incl. quant "
                f"{per_gemm[-1]['incl_quant_tflops']:7.1f}")
        quant_cold = []
        ceil = copy_ceiling(hp, args.reps) if args.quant_ceiling else {}
        for i, (op, st) in enumerate(zip(hp.ops, sw)):
            if op.kind == "gemm":
                continue
            gbs = op.bytes / (st["median"] * 1e-6) / 1e9
            quant_cold.append({"call": op.label, "median_us": round(st["median"], 2),
                               "p10_us": round(st["p10"], 2), "p90_us": round(st["p90"], 2),
                               "gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)})
            extra = ""
            if i in ceil:
                cu, cb = ceil[i]
                quant_cold[-1].update({"copy_same_input_us": round(cu, 2),
                                       "copy_gbs": round(cb / (cu * 1e-6) / 1e9, 1),
                                       "copy_time_over_quant_time": round(cu / st["median"], 3)})
                extra = (f"; copy of the input volume {cu:6.1f} us "
                         f"({cb / (cu * 1e-6) / 1e9:6.0f} GB/s)")
            log(f"[bench] {op.label:22s} median {st['median']:7.1f} us  {gbs:7.1f} GB/s "
                f"({100 * gbs / HBM_PEAK_GBS:.1f} % of HBM){extra}")
            if op.kind == "weight_quant":
                weight_quant = (weight_quant or 0.0) + st["median"]
        if qroof is not None:
            qroof["cold_per_call"] = quant_cold
    # ---- phase 5: clock window ------------------------------------------------
    clock = None
    if args.clock_window > 0:
        clocks = ClockSampler()
        torch.cuda.synchronize()
        clocks.start()
        t_c0 = time.perf_counter()
        n_win = 0
        while time.perf_counter() - t_c0 < args.clock_window:
            for _ in range(10):
                hp.run()
            torch.cuda.synchronize()
            n_win += 10
        t_c1 = time.perf_counter()
        clocks.stop()
        clock = clocks.summary(t_c0, t_c1)
    if clock is not None:
        clock["window_s"] = round(t_c1 - t_c0, 2)
        clock["window_tflops"] = round(flops_step * n_win / (t_c1 - t_c0) / 1e12, 1)
        log(f"[bench] clock window: {n_win} passes, {clock['window_tflops']} TFLOP/s, gfx "
            f"{clock['gfx_mhz_median']} MHz median, {clock['socket_power_w_median']} W")
        if clock.get("gfx_mhz_median"):
            # the same GEMM rate against the FP8 peak at the clock the chip actually ran
            peak_clk = FP8_DENSE_PEAK_TFLOPS * clock["gfx_mhz_median"] / PEAK_GFX_MHZ
            roofline["clock_adjusted"] = {
                "gfx_mhz_median": clock["gfx_mhz_median"], "peak": round(peak_clk, 1),
                "frac": round(roofline["achieved"] / peak_clk, 4),
                "note": "peak scaled by the median graphics clock of the clock window / 2400 MHz"}

    for i, op in enumerate(hp.ops):
        if op.kind == "gemm":
            log(f"[bench] in-pass {op.label:15s} {mean_us[i]:8.1f} us (min {spread[i][0]:.1f}, "
                f"max {spread[i][1]:.1f})  {op.flops / (mean_us[i] * 1e-6) / 1e12:7.1f} TFLOP/s")
    gemm_ms = sum(mean_us[i] for i, op in enumerate(hp.ops) if op.kind == "gemm") / 1e3
    log(f"[bench] GEMM time {gemm_ms:.3f} ms of {statistics.median(step_ms):.3f} ms per step")

    bf16 = None
    if not args.no_bf16_baseline:
        bf16 = bf16_baseline(tensors, wl, max(args.steps // 3, 3), value)

    smm = None
    if args.scaled_mm_baseline:
        smm = scaled_mm_baseline(hp, min(args.reps, 20))

    accuracy = None
    if args.accuracy:
        accuracy = accuracy_report(tensors, wl, hp)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        cpu = cpu_baseline(wl.name, args.cpu_tokens, args.scales)

    wq_amortised = None
    if weight_quant is not None:
        wq_amortised = {"weight_quant_us_per_step": round(weight_quant, 2),
                        "amortised_us_per_microbatch": round(weight_quant / MICROBATCHES_PER_STEP, 3),
                        "microbatches_per_optimizer_step": MICROBATCHES_PER_STEP,
                        "value_with_amortised_weight_quant": round(
                            flops_step / ((statistics.median(step_ms) - weight_quant * 1e-3
                                           + weight_quant * 1e-3 / MICROBATCHES_PER_STEP) * 1e-3)
                            / 1e12, 2)}

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "step_ms": {"median": round(statistics.median(step_ms), 4),
                    "p10": round(pct(step_ms, 10), 4), "p90": round(pct(step_ms, 90), 4),
                    "source": "HIP events around each timed pass"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8_e4m3 (fp32 accumulate, bf16 out)" if args.scales == "fp32" else
                  f"fp8_e4m3 with E8M0 scales, {args.scales} (fp32 accumulate, bf16 out)"),
        "data": "synthetic",
        "pct_fp8_peak": round(100 * value / FP8_DENSE_PEAK_TFLOPS, 2),
        "config": {
            "workload": wl.name,
            "tokens": wl.tokens,
            "linears": {L.name: [L.in_features, L.out_features] for L in wl.linears},
            "roles": wl.roles,
            "gemms_per_step": len(wl.gemms),
            "tflop_per_step": round(flops_step / 1e12, 4),
            "includes": "weight, activation, gradient and token-axis quantisers + every GEMM",
        },
        "roofline": roofline,
        "quant_roofline": qroof,
        "per_gemm": per_gemm,
        "weight_quant": wq_amortised,
        "clock": clock,
        "cpu_baseline": cpu,
        "bf16_baseline": bf16,
    }
    if smm is not None:
        line["scaled_mm_baseline"] = smm
    if accuracy is not None:
        line["accuracy"] = accuracy
    if graph is not None:
        line["graph_replay"] = graph
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
