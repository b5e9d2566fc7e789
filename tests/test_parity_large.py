"""The largest sizes the entry points accept, against the oracle on sampled
outputs: byte offsets past 2**31 in the quantisers, the largest token-block
grid of the dual quantiser, and the largest leading dimension the GEMM
addresses (4 MiB rows, K = 2**22).  Inputs are drawn on the device from a
seeded generator; the sampled rows, groups and outputs are copied back and
checked element by element (codes and scale bits exactly, GEMM outputs
under the gate of tests/gate.py)."""
import numpy as np
import pytest
import torch

import gate
import oracle
from workloads import to_numpy_input

pytestmark = pytest.mark.gpu

import blockwise_fp8_gemm_bfp8_amd as bfp8  # noqa: E402


def same_codes(got_q, got_s, exp_q, exp_s, what):
    gq = got_q.cpu().numpy()
    gs = got_s.cpu().numpy()
    assert np.array_equal(gq, exp_q), f"{what}: codes differ"
    assert np.array_equal(gs.view(np.uint32), exp_s.view(np.uint32)), f"{what}: scales differ"


def release(*ts):
    del ts
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_quantize_act_codes_past_2gib():
    """4 GiB of codes (8 GiB of bf16 input): rows near the end sit past
    2**31 bytes from the start of both buffers."""
    rows, cols = 1 << 21, 2048
    g = torch.Generator(device="cuda").manual_seed(12)
    x = torch.randn((rows, cols), device="cuda", dtype=torch.bfloat16, generator=g)
    q, s = bfp8.quantize_act(x)
    torch.cuda.synchronize()
    for r in (0, 1, (1 << 20) + 7, rows - 2, rows - 1):
        eq, es = oracle.quantize_act(to_numpy_input(x[r:r + 1].cpu()))
        same_codes(q[r:r + 1], s[r:r + 1], eq, es, f"row {r}")
    release(x, q, s)


def test_quantize_act_dual_largest_token_grid():
    """65535 token blocks (8388480 tokens, the largest grid) x 256 channels:
    the transposed codes of the last channel start past 2**31 bytes."""
    rows, cols = 65535 * 128, 256
    g = torch.Generator(device="cuda").manual_seed(13)
    x = torch.randn((rows, cols), device="cuda", dtype=torch.bfloat16, generator=g)
    q, s, qt, st = bfp8.quantize_act_dual(x)
    torch.cuda.synchronize()
    for r in (0, 1, 4194307, rows - 1):
        eq, es = oracle.quantize_act(to_numpy_input(x[r:r + 1].cpu()))
        same_codes(q[r:r + 1], s[r:r + 1], eq, es, f"row {r}")
    for b in (0, 1, 32768, 65534):
        eqt, est = oracle.quantize_act_transposed(to_numpy_input(x[128 * b:128 * b + 128].cpu()))
        same_codes(qt[:, 128 * b:128 * b + 128], st[:, b:b + 1], eqt, est, f"token block {b}")
    release(x, q, s, qt, st)


def random_codes(shape, g):
    q = torch.empty(shape, dtype=torch.uint8, device="cuda").random_(0, 256, generator=g)
    q[(q & 0x7F) == 0x7F] = 0x7E  # no NaN codes
    return q


def test_gemm_largest_leading_dimension():
    """NT with K = 2**22: lda = ldb = 4 MiB, the largest leading dimension
    the GEMM addresses; 2 x 2 tiles with ragged edges, split along K."""
    M, N, K = 260, 264, 1 << 22
    g = torch.Generator(device="cuda").manual_seed(11)
    qa = random_codes((M, K), g)
    qb = random_codes((N, K), g)
    sa = torch.rand((M, K // 128), device="cuda", generator=g) + 0.5
    sb = torch.rand((N, K // 128), device="cuda", generator=g) + 0.5
    C = bfp8.gemm("NT", qa, sa, qb, sb, "act", "act")
    torch.cuda.synchronize()
    rows, cols = [0, 1, 255, 256, 259], [0, 3, 255, 256, 263]
    ac, asc = oracle.logical_operand(qa[rows].cpu().numpy(), sa[rows].cpu().numpy(), "A", "N", "act")
    bc, bsc = oracle.logical_operand(qb[cols].cpu().numpy(), sb[cols].cpu().numpy(), "B", "T", "act")
    got = C.float().cpu().numpy()[np.ix_(rows, cols)]
    gate.check(got, ac, asc, bc, bsc, ("largest leading dimension", M, N, K))
    release(qa, qb, sa, sb, C)
