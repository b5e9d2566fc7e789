"""Benchmark: blockwise-FP8 linear layers (quantise + GEMM) on one MI355X.

A step is one full pass of the hot path over one batch of synthetic input:
for each of the four linears of a Puro-2B decoder layer at M = 16384 tokens
(QKV 2048->4096, o_proj 2048->2048, gate/up 2048->12288, down 6144->2048):
weight quantisation, activation quantisation and the fprop GEMM; gradient
quantisation and the dgrad GEMM; token-axis quantisation of dY and X and the
wgrad GEMM -- 12 GEMMs, 4.95 TFLOP.  Inputs are resident in HBM before the
timed region.  Prints ONE JSON line on stdout; details go to stderr.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--scales fp32|mx128|mx32] [--no-cpu-baseline] [--no-bf16-baseline]
                  [--copy-calibration]

--scales picks the scale format of the pass: fp32 (float32 amax/448 scales,
promotion on the VALU; the default and the headline), mx128 (the same groups
with power-of-two E8M0 scales applied by the scaled MFMA) or mx32 (MXFP8,
1x32 power-of-two groups).  The line also carries `bf16_baseline`: the same
12 GEMMs on the unquantised bf16 tensors through torch.matmul (hipBLASLt),
timed the same way, for the FP8-over-BF16 ratio.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "blockwise-FP8 GEMM TFLOP/s incl. quantize at Puro-2B shapes; % FP8 MFMA peak"
FP8_DENSE_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 MFMA, published
HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "layer_fwd_bwd_m16384"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_traffic.json")
GEMM_SOURCE = os.path.join(ROOT, "blockwise_fp8_gemm_bfp8_amd", "csrc", "gemm.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


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


def cpu_baseline(workload_name, tokens_sample, scales="fp32"):
    """The oracle (numpy, float64 GEMM) on the same workload with M cut to
    `tokens_sample` tokens: every quantiser and all GEMMs of the step."""
    import numpy as np

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
    }


def bf16_baseline(tensors, wl, steps, fp8_value):
    """The step's 12 GEMMs on the unquantised bf16 tensors via torch.matmul
    (hipBLASLt), no quantisation: fprop X W^T, dgrad dY W, wgrad dY^T X."""
    import torch

    # every operand contiguous: the transposes W^T and dY^T are materialised
    # once, outside the timed steps, so each product is a plain row-major
    # matmul (transposed-view bf16 products are avoided altogether: their
    # batched form has faulted on this software stack)
    lin = [(tensors["x." + L.name], tensors["w." + L.name], tensors["dy." + L.name],
            tensors["w." + L.name].t().contiguous(), tensors["dy." + L.name].t().contiguous())
           for L in wl.linears]

    def step():
        for x, _, _, wt, _ in lin:
            torch.matmul(x, wt)
        for x, w, dy, _, dyt in lin:
            torch.matmul(dy, w)
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
            "kind": "the same 12 GEMMs in bf16 via torch.matmul (hipBLASLt), unquantised",
            "fp8_over_bf16": round(fp8_value / value, 3)}


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
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library has no "
              "multi-GPU path -- each GPU runs the same data-parallel step independently.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from blockwise_fp8_gemm_bfp8_amd import build as _build

    if not os.path.exists(_build.LIB_PATH):
        _build.build()
    from blockwise_fp8_gemm_bfp8_amd.hotpath import HotPath
    from workloads import WORKLOADS, make_inputs

    wl = WORKLOADS[args.workload]
    log(f"[bench] workload {wl.name}: generating inputs")
    tensors = {k: v.cuda() for k, v in make_inputs(wl.name).items()}
    hp = HotPath(tensors, [L.name for L in wl.linears], wl.roles, scales=args.scales)
    flops_step = wl.flops
    # HotPath.run launches the GEMMs in this order:
    order = [g for g in wl.gemms if g.role == "fprop"]
    for L in wl.linears:
        order += [g for g in wl.gemms if g.linear is L and g.role in ("dgrad", "wgrad")]
    gemm_flops = [g.flops for g in order]

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

    log(f"[bench] timing {args.steps} steps")
    hp.gemm_events = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        hp.run()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed / args.steps * 1e3
    value = flops_step / (elapsed / args.steps) / 1e12

    durs = [s.elapsed_time(e) for s, e in hp.gemm_events]  # ms
    n_g = len(gemm_flops)
    per_gemm = {}
    for i, d in enumerate(durs):
        per_gemm.setdefault(i % n_g, []).append(d)
    total_gemm_ms = sum(durs)
    total_gemm_flops = sum(gemm_flops) * args.steps
    avg_launch_ms = total_gemm_ms / len(durs)
    avg_flops = sum(gemm_flops) / n_g
    achieved = avg_flops / (avg_launch_ms * 1e-3) / 1e12
    traffic = load_traffic()
    roofline = {
        "kernel": ("gemm_kernel (blockwise FP8 GEMM; mean over the step's GEMM launches)"
                   if args.scales == "fp32" else
                   f"gemm_kernel, E8M0 instantiation ({args.scales}; mean over the step's GEMM "
                   "launches)"),
        "bound": "mfma",
        "achieved": round(achieved, 1),
        "peak": FP8_DENSE_PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / FP8_DENSE_PEAK_TFLOPS, 4),
        "traffic": traffic,
        "avg_launch_us": round(avg_launch_ms * 1e3, 2),
    }
    for i, g in enumerate(order):
        d = sum(per_gemm[i]) / len(per_gemm[i])
        log(f"[bench] {g.linear.name:8s} {g.role:5s} {g.layout} M,N,K={g.mnk}: "
            f"{d * 1e3:8.1f} us  {g.flops / (d * 1e-3) / 1e12:7.1f} TFLOP/s")
    log(f"[bench] GEMM time {total_gemm_ms / args.steps:.3f} ms of {ms_per_step:.3f} ms per step")

    bf16 = None
    if not args.no_bf16_baseline and set(wl.roles) == {"fprop", "dgrad", "wgrad"}:
        bf16 = bf16_baseline(tensors, wl, max(args.steps // 3, 3), value)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        cpu = cpu_baseline(wl.name, args.cpu_tokens, args.scales)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
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
            "gemms_per_step": len(wl.gemms),
            "tflop_per_step": round(flops_step / 1e12, 4),
            "includes": "weight, activation, gradient and token-axis quantisers + 12 GEMMs",
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "bf16_baseline": bf16,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
