"""The training pass captured into a HIP graph: every kernel of a pass is an
ordinary launch on the current stream with preallocated buffers (no
allocation, no memset), so the pass can be captured once and replayed.  Each
replay, with eager work and synchronisations between the replays, must
reproduce the eager pass byte for byte."""
import pytest
import torch

from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

from blockwise_fp8_gemm_bfp8_amd.hotpath import HotPath  # noqa: E402

OUTPUTS = ("wq", "ws", "xq", "xs", "xqt", "xst", "y", "dyq", "dys", "dyqt", "dyst", "dx", "dw")


def snapshot(hp):
    return [(L.name, k, L.buf[k].clone()) for L in hp.layers for k in OUTPUTS if k in L.buf]


@pytest.mark.parametrize("scales", ["fp32", "mx128"])
def test_layer_pass_graph_replays_match_eager(scales):
    wl = WORKLOADS["layer_fwd_bwd_m16384"]
    t = {k: v.cuda() for k, v in make_inputs(wl.name).items()}
    hp = HotPath(t, [L.name for L in wl.linears], wl.roles, scales=scales)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        hp.run()                              # warm-up off the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    hp.run()                                  # eager reference
    torch.cuda.synchronize()
    ref = snapshot(hp)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        hp.run()
    torch.cuda.synchronize()
    a = torch.randn((2048, 2048), device="cuda")
    for rep in range(3):
        for L in hp.layers:                   # clear every output eagerly
            for k in OUTPUTS:
                if k in L.buf:
                    L.buf[k].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (name, k, want), (_, _, got) in zip(ref, snapshot(hp)):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), (scales, rep, name, k)
        a = a @ a.t() / 2048.0                # unrelated eager work between replays
        torch.cuda.synchronize()
    del g, hp, t
    torch.cuda.empty_cache()
