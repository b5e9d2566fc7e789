"""Whole hot path at the workload shapes, in the launch configuration the
benchmark times (blockwise_fp8_gemm_bfp8_amd.hotpath.HotPath), against the
oracle on sampled outputs.

For every GEMM the oracle quantises only the rows/channels it needs (1x128
groups are independent across rows, token groups across channels; weights are
quantised whole), dequantises in float64 and multiplies; the GPU output at
the same (m, n) must be within the 1e-2 tolerance, and the GPU's codes and
scales for those rows must match the oracle's bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS, make_inputs, to_numpy_input

pytestmark = pytest.mark.gpu

from blockwise_fp8_gemm_bfp8_amd.hotpath import HotPath  # noqa: E402

TOL = 1e-2


def sample(n, k, rng):
    if n <= k:
        return np.arange(n)
    return np.sort(rng.choice(n, k, replace=False))


def deq_rows_act(q, s):
    """float64 dequantisation of act-mode rows [r][K] with scales [r][K/128]."""
    return oracle.dequantize_operand(q, s, "A", "N", "act")


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_hot_path(name):
    wl = WORKLOADS[name]
    t = make_inputs(name)
    dev = {k: v.cuda() for k, v in t.items()}
    hp = HotPath(dev, [L.name for L in wl.linears], wl.roles)
    hp.run()
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    for L, st in zip(wl.linears, hp.layers):
        b = st.buf
        x = to_numpy_input(t["x." + L.name])
        w = to_numpy_input(t["w." + L.name])
        wq, ws = oracle.quantize_weight(w)
        assert np.array_equal(b["wq"].cpu().numpy(), wq)
        assert np.array_equal(b["ws"].cpu().numpy().view(np.uint32), ws.view(np.uint32))
        W = oracle.dequantize_operand(wq, ws, "B", "T", "block")  # logical [in][out]
        M = wl.tokens
        if "fprop" in wl.roles:
            rows = sample(M, 192, rng)
            cols = sample(L.out_features, 256, rng)
            xq, xs = oracle.quantize_act(x[rows])
            assert np.array_equal(b["xq"].cpu().numpy()[rows], xq)
            R = deq_rows_act(xq, xs) @ W[:, cols]
            C = b["y"].float().cpu().numpy()[np.ix_(rows, cols)]
            err = oracle.rel_error(C, R)
            assert err <= TOL, (name, L.name, "fprop", err)
        if "dgrad" in wl.roles:
            dy = to_numpy_input(t["dy." + L.name])
            rows = sample(M, 192, rng)
            cols = sample(L.in_features, 256, rng)
            dq, ds = oracle.quantize_act(dy[rows])
            assert np.array_equal(b["dyq"].cpu().numpy()[rows], dq)
            # dgrad B is W's codes as stored, [K=out][N=in]: logical B = Wdeq^T
            R = deq_rows_act(dq, ds) @ W.T[:, cols]
            C = b["dx"].float().cpu().numpy()[np.ix_(rows, cols)]
            err = oracle.rel_error(C, R)
            assert err <= TOL, (name, L.name, "dgrad", err)
        if "wgrad" in wl.roles:
            dy = to_numpy_input(t["dy." + L.name])
            rows = sample(L.out_features, 96, rng)   # output channels of dW
            cols = sample(L.in_features, 96, rng)    # input channels of dW
            aq, as_ = oracle.quantize_act_transposed(np.ascontiguousarray(dy[:, rows]))
            bq, bs = oracle.quantize_act_transposed(np.ascontiguousarray(x[:, cols]))
            assert np.array_equal(b["dyqt"].cpu().numpy()[rows], aq)
            assert np.array_equal(b["xqt"].cpu().numpy()[cols], bq)
            R = deq_rows_act(aq, as_) @ deq_rows_act(bq, bs).T
            C = b["dw"].float().cpu().numpy()[np.ix_(rows, cols)]
            err = oracle.rel_error(C, R)
            assert err <= TOL, (name, L.name, "wgrad", err)
    del hp, dev
    torch.cuda.empty_cache()


@pytest.mark.parametrize("scales", ["mx128", "mx32"])
def test_layer_hot_path_power_of_two(scales):
    """The full decoder-layer pass (M = 16384) with power-of-two scales, in
    the configuration `bench.py --scales` times, against the E8M0 oracle on
    sampled outputs (codes and scale bytes of the sampled rows bit-exact)."""
    name = "layer_fwd_bwd_m16384"
    wl = WORKLOADS[name]
    t = make_inputs(name)
    dev = {k: v.cuda() for k, v in t.items()}
    hp = HotPath(dev, [L.name for L in wl.linears], wl.roles, scales=scales)
    hp.run()
    torch.cuda.synchronize()
    grp = 32 if scales == "mx32" else 128
    mode = "mx32" if grp == 32 else "act"
    rng = np.random.default_rng(11)
    M = wl.tokens
    for L, st in zip(wl.linears, hp.layers):
        b = st.buf
        x = to_numpy_input(t["x." + L.name])
        w = to_numpy_input(t["w." + L.name])
        dy = to_numpy_input(t["dy." + L.name])
        if grp == 32:
            wq, ws = oracle.quantize_mx_act(w, 32)
            wqt, wst = oracle.quantize_mx_act_transposed(w, 32)
            assert np.array_equal(b["wqt"].cpu().numpy(), wqt)
            assert np.array_equal(b["wst"].cpu().numpy(), wst)
            Wf = oracle.dequantize_mx_operand(wq, ws, "B", "T", "mx32")     # [in][out]
            Wd = oracle.dequantize_mx_operand(wqt, wst, "B", "T", "mx32")   # [out][in]
        else:
            wq, ws = oracle.quantize_mx_weight(w)
            Wf = oracle.dequantize_mx_operand(wq, ws, "B", "T", "block")
            Wd = Wf.T
        assert np.array_equal(b["wq"].cpu().numpy(), wq)
        assert np.array_equal(b["ws"].cpu().numpy(), ws)
        rows = sample(M, 160, rng)
        cols = sample(L.out_features, 192, rng)
        xq, xs = oracle.quantize_mx_act(x[rows], grp)
        assert np.array_equal(b["xq"].cpu().numpy()[rows], xq)
        assert np.array_equal(b["xs"].cpu().numpy()[rows], xs)
        R = oracle.dequantize_mx_operand(xq, xs, "A", "N", mode) @ Wf[:, cols]
        err = oracle.rel_error(b["y"].float().cpu().numpy()[np.ix_(rows, cols)], R)
        assert err <= TOL, (scales, L.name, "fprop", err)
        cols = sample(L.in_features, 192, rng)
        dq, ds = oracle.quantize_mx_act(dy[rows], grp)
        assert np.array_equal(b["dyq"].cpu().numpy()[rows], dq)
        R = oracle.dequantize_mx_operand(dq, ds, "A", "N", mode) @ Wd[:, cols]
        err = oracle.rel_error(b["dx"].float().cpu().numpy()[np.ix_(rows, cols)], R)
        assert err <= TOL, (scales, L.name, "dgrad", err)
        orow = sample(L.out_features, 64, rng)
        icol = sample(L.in_features, 64, rng)
        aq, as_ = oracle.quantize_mx_act_transposed(np.ascontiguousarray(dy[:, orow]), grp)
        bq, bs = oracle.quantize_mx_act_transposed(np.ascontiguousarray(x[:, icol]), grp)
        assert np.array_equal(b["dyqt"].cpu().numpy()[orow], aq)
        assert np.array_equal(b["xst"].cpu().numpy()[icol], bs)
        R = (oracle.dequantize_mx_operand(aq, as_, "A", "N", mode)
             @ oracle.dequantize_mx_operand(bq, bs, "A", "N", mode).T)
        err = oracle.rel_error(b["dw"].float().cpu().numpy()[np.ix_(orow, icol)], R)
        assert err <= TOL, (scales, L.name, "wgrad", err)
    del hp, dev
    torch.cuda.empty_cache()


def test_bf16_baseline_gemm_matches_float64():
    """The BF16 comparison point of the benchmark (torch.matmul on the
    unquantised bf16 tensors, hipBLASLt, every operand contiguous): within
    bf16 output rounding plus fp32 accumulation of the float64 product of
    the same bf16 values, for the fprop, dgrad and wgrad products."""
    t = make_inputs("qkv_fprop_m8192")
    x = t["x.qkv"][:512].cuda()
    w = t["w.qkv"][:384].cuda()
    dy = (torch.randn((512, 384), generator=torch.Generator().manual_seed(3)) * 1e-3).to(
        torch.bfloat16).cuda()
    xn, wn, dyn = (v.float().cpu().numpy().astype(np.float64) for v in (x, w, dy))
    wt = w.t().contiguous()
    dyt = dy.t().contiguous()
    for got, R in ((torch.matmul(x, wt), xn @ wn.T), (torch.matmul(dy, w), dyn @ wn),
                   (torch.matmul(dyt, x), dyn.T @ xn)):
        err = oracle.rel_error(got.float().cpu().numpy(), R)
        assert err <= 2.0 ** -7, err
