"""bfp8_gemm_static_scratch: the GEMM entry point that allocates nothing (its
split-K partials live in the library's static device array), called through
the C ABI and checked against bfp8_gemm with a caller workspace -- bit for
bit, since both take the same split plan and the same reduction order -- and
against the oracle under the parity gate, on two calls in a row, the second
smaller."""
import ctypes

import numpy as np
import pytest
import torch

import gate
import oracle

pytestmark = pytest.mark.gpu

import blockwise_fp8_gemm_bfp8_amd as bfp8  # noqa: E402


def codes(shape, g):
    q = torch.empty(shape, dtype=torch.uint8, device="cuda").random_(0, 256, generator=g)
    q[(q & 0x7F) == 0x7F] = 0x7E
    return q


def call_static(qa, sa, qb, sb, out):
    M, K = qa.shape
    N = qb.shape[0]
    return bfp8.lib().bfp8_gemm_static_scratch(
        bfp8.LAYOUTS["NT"], M, N, K, ctypes.c_void_p(qa.data_ptr()), qa.stride(0),
        ctypes.c_void_p(sa.data_ptr()), bfp8.MODES["act"], ctypes.c_void_p(qb.data_ptr()),
        qb.stride(0), ctypes.c_void_p(sb.data_ptr()), bfp8.MODES["act"],
        ctypes.c_void_p(out.data_ptr()), out.stride(0),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("shapes", [[(2048, 2048, 16384), (1024, 512, 16384)],
                                    [(2048, 2048, 16384), (8448, 2048, 4096)]])
def test_static_scratch_gemm_matches_workspace_gemm(shapes):
    """Every tile split (2048 x 2048 and 1024 x 512 at K = 16384), or 256
    whole tiles and only the last row of tiles split (8448 x 2048 x 4096);
    each pair: two calls in a row, the second with fewer input bytes."""
    g = torch.Generator(device="cuda").manual_seed(5)
    for M, N, K in shapes:
        need = bfp8.gemm_workspace_bytes("NT", "act", "act", M, N, K)
        assert 0 < need <= bfp8.STATIC_SCRATCH_BYTES, need   # the split-K path, within the array
        qa, qb = codes((M, K), g), codes((N, K), g)
        sa = torch.rand((M, K // 128), device="cuda", generator=g) + 0.5
        sb = torch.rand((N, K // 128), device="cuda", generator=g) + 0.5
        out = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
        assert call_static(qa, sa, qb, sb, out) == 0
        ref = bfp8.gemm("NT", qa, sa, qb, sb, "act", "act")   # allocates its workspace
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), (M, N, K)
        rows = np.r_[0:M:M // 16, M - 64:M]   # the last rows lie in split tiles
        ac, asc = oracle.logical_operand(qa[rows].cpu().numpy(), sa[rows].cpu().numpy(),
                                         "A", "N", "act")
        bc, bsc = oracle.logical_operand(qb.cpu().numpy(), sb.cpu().numpy(), "B", "T", "act")
        gate.check(out.float().cpu().numpy()[rows], ac, asc, bc, bsc, ("static scratch", M, N, K))


def test_static_scratch_rejects_partials_beyond_the_array():
    """3072 x 4096 x 65536 (12 x 16 tiles, each split 4 ways along K): 192 MiB
    of split-K partials, more than the array holds -> BFP8_ERR_WORKSPACE
    before any launch; the output is untouched."""
    M, N, K = 3072, 4096, 65536
    assert bfp8.gemm_workspace_bytes("NT", "act", "act", M, N, K) > bfp8.STATIC_SCRATCH_BYTES
    qa = torch.zeros((M, K), dtype=torch.uint8, device="cuda")
    qb = torch.zeros((N, K), dtype=torch.uint8, device="cuda")
    sa = torch.ones((M, K // 128), device="cuda")
    sb = torch.ones((N, K // 128), device="cuda")
    out = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
    assert call_static(qa, sa, qb, sb, out) == 7   # BFP8_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert (out == 3.0).all()
