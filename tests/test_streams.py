"""The library keeps no state between calls: the same work launched on two
streams at once, quantisers and GEMMs interleaved (split-K with each call's
own workspace included), gives the bytes a sequential run gives."""
import pytest
import torch

pytestmark = pytest.mark.gpu

import blockwise_fp8_gemm_bfp8_amd as bfp8  # noqa: E402


def job(x, w, dy):
    """fprop, dgrad and split-K wgrad of one linear; returns every output."""
    xq, xs, xqt, xst = bfp8.quantize_act_dual(x)
    wq, ws = bfp8.quantize_weight(w)
    dq, ds, dqt, dst = bfp8.quantize_act_dual(dy)
    y = bfp8.gemm("NT", xq, xs, wq, ws, "act", "block")
    dx = bfp8.gemm("NN", dq, ds, wq, ws, "act", "block")
    dw = bfp8.gemm("NT", dqt, dst, xqt, xst, "act", "act")
    return [xq, xs, xqt, xst, wq, ws, dq, ds, dqt, dst, y, dx, dw]


def inputs(seed, M, K, N):
    g = torch.Generator(device="cuda").manual_seed(seed)
    x = torch.randn((M, K), device="cuda", generator=g).to(torch.bfloat16)
    w = (torch.randn((N, K), device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    dy = (torch.randn((M, N), device="cuda", generator=g) * 1e-3).to(torch.bfloat16)
    return x, w, dy


def test_two_streams_match_sequential():
    a = inputs(1, 4096, 1024, 768)      # wgrad 768 x 1024 x 4096 runs split along K
    b = inputs(2, 2048, 2048, 1536)
    torch.cuda.synchronize()
    ref_a, ref_b = job(*a), job(*b)
    torch.cuda.synchronize()
    ref_a = [t.clone() for t in ref_a]
    ref_b = [t.clone() for t in ref_b]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        with torch.cuda.stream(s1):
            out_a = job(*a)
        with torch.cuda.stream(s2):
            out_b = job(*b)
        torch.cuda.synchronize()
        for want, got in zip(ref_a + ref_b, out_a + out_b):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8))


def job_mx(x, w, dy):
    """The same linear with power-of-two scales (the persistent GEMM kernel:
    each call launches one workgroup per CU walking its tiles)."""
    xq, xs, xqt, xst = bfp8.quantize_mx_act_dual(x)
    wq, ws = bfp8.quantize_mx_weight(w)
    dq, ds, dqt, dst = bfp8.quantize_mx_act_dual(dy)
    y = bfp8.gemm_mx("NT", xq, xs, wq, ws, "act", "block")
    dx = bfp8.gemm_mx("NN", dq, ds, wq, ws, "act", "block")
    dw = bfp8.gemm_mx("NT", dqt, dst, xqt, xst, "act", "act")
    return [xq, xs, xqt, xst, wq, ws, dq, ds, dqt, dst, y, dx, dw]


def test_two_streams_match_sequential_power_of_two():
    a = inputs(3, 8192, 1024, 2048)     # fprop 8192 x 2048: 256 tiles; wgrad split along K
    b = inputs(4, 4096, 2048, 4608)     # fprop 4096 x 4608: 288 tiles, more than one per CU
    torch.cuda.synchronize()
    ref_a, ref_b = job_mx(*a), job_mx(*b)
    torch.cuda.synchronize()
    ref_a = [t.clone() for t in ref_a]
    ref_b = [t.clone() for t in ref_b]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        with torch.cuda.stream(s1):
            out_a = job_mx(*a)
        with torch.cuda.stream(s2):
            out_b = job_mx(*b)
        torch.cuda.synchronize()
        for want, got in zip(ref_a + ref_b, out_a + out_b):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8))
