"""The fence-free HIP events that time the GEMMs of a pass
(blockwise_fp8_gemm_bfp8_amd.hotpath.TimingEvent): they record on the
current stream and measure what torch's own events measure."""
import pytest
import torch

pytestmark = pytest.mark.gpu

from blockwise_fp8_gemm_bfp8_amd.hotpath import TimingEvent  # noqa: E402


def test_timing_event_brackets_a_kernel():
    a = torch.randn((4096, 4096), device="cuda")
    b = torch.randn((4096, 4096), device="cuda")
    torch.matmul(a, b)
    torch.cuda.synchronize()
    s, e = TimingEvent(), TimingEvent()
    ts, te = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts.record()
    s.record()
    for _ in range(10):
        torch.matmul(a, b)
    e.record()
    te.record()
    torch.cuda.synchronize()
    ms, ref = s.elapsed_time(e), ts.elapsed_time(te)
    assert ms > 0
    # both pairs bracket the same ten products (theirs one record wider on each side)
    assert abs(ms - ref) <= 0.2 * ref + 0.05, (ms, ref)
