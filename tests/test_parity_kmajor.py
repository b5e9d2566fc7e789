"""K-block-major scale layout (BFP8_SCALE_1x128_KMAJOR and the _kmajor
quantisers): the same codes byte for byte, the same scales transposed, and
GEMM outputs bit-identical to the default layout -- only where the scales sit
in memory changes.  Shapes include ragged row / channel extents and both
tile widths of the dual quantiser (128 and 256 channels)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import blockwise_fp8_gemm_bfp8_amd as bfp8  # noqa: E402


def rand(shape, seed, dtype):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(shape, generator=g) * torch.exp(torch.randn(shape, generator=g))
    return x.to(dtype).cuda()


def same(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


DTYPES = [torch.bfloat16, torch.float32]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", [(256, 512), (300, 384), (1024, 2048), (1, 128)])
def test_act_kmajor(dtype, shape):
    x = rand(shape, sum(shape), dtype)
    q, s = bfp8.quantize_act(x)
    qk, sk = bfp8.quantize_act_kmajor(x)
    torch.cuda.synchronize()
    assert same(q, qk) and same(s.t(), sk)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", [(256, 200), (512, 384), (2048, 6144)])
def test_transposed_kmajor(dtype, shape):
    x = rand(shape, sum(shape) + 1, dtype)
    qt, st = bfp8.quantize_act_transposed(x)
    qtk, stk = bfp8.quantize_act_transposed_kmajor(x)
    torch.cuda.synchronize()
    assert same(qt, qtk) and same(st.t(), stk)


@pytest.mark.parametrize("dtype,shape", [(torch.bfloat16, (256, 256)), (torch.bfloat16, (384, 6144)),
                                         (torch.bfloat16, (1024, 2048)), (torch.float32, (256, 384))])
def test_dual_kmajor(dtype, shape):
    x = rand(shape, sum(shape) + 2, dtype)
    q, s, qt, st = bfp8.quantize_act_dual(x)
    qk, sk, qtk, stk = bfp8.quantize_act_dual_kmajor(x)
    torch.cuda.synchronize()
    assert same(q, qk) and same(qt, qtk)
    assert same(s.t(), sk) and same(st.t(), stk)


@pytest.mark.parametrize("dtype,shape", [(torch.bfloat16, (256, 256)), (torch.bfloat16, (384, 6144)),
                                         (torch.float32, (256, 384))])
def test_mx_dual_kmajor(dtype, shape):
    x = rand(shape, sum(shape) + 3, dtype)
    q, s, qt, st = bfp8.quantize_mx_act_dual(x, 128)
    qk, sk, qtk, stk = bfp8.quantize_mx_act_dual_kmajor(x)
    torch.cuda.synchronize()
    assert same(q, qk) and same(qt, qtk)
    assert same(s.t(), sk) and same(st.t(), stk)


def codes(shape, g):
    q = torch.empty(shape, dtype=torch.uint8, device="cuda").random_(0, 256, generator=g)
    q[(q & 0x7F) == 0x7F] = 0x7E
    return q


@pytest.mark.parametrize("layout,ma,mb", [("NT", "act", "block"), ("NT", "act", "act"),
                                          ("NT", "block", "act"), ("NN", "act", "block"),
                                          ("NN", "act", "act"), ("TN", "act", "act")])
@pytest.mark.parametrize("mx", [False, True])
def test_gemm_kmajor_scales_bitwise(layout, ma, mb, mx):
    M, N, K = 304, 528, 1024   # ragged against the 256 tile, rows 16-byte aligned
    g = torch.Generator(device="cuda").manual_seed(17)
    qa = codes((M, K) if layout[0] == "N" else (K, M), g)
    qb = codes((K, N) if layout[1] == "N" else (N, K), g)

    def scales(rows, role_n, mode):
        # default-layout scale tensor and its K-block-major form
        KB = K // 128
        if mode == "block":
            shape = ((rows + 127) // 128, KB) if role_n else (KB, (rows + 127) // 128)
        else:
            shape = (rows, KB) if role_n else (KB, rows)
        if mx:
            s = torch.randint(120, 135, shape, dtype=torch.uint8, device="cuda", generator=g)
            sd = bfp8._scale_bytes(*shape, "cuda").copy_(s)
        else:
            sd = (torch.rand(shape, device="cuda", generator=g) + 0.5).contiguous()
        if mode == "block":
            return sd, sd, mode
        kmj = sd.t().contiguous() if role_n else sd
        if mx:
            kmj = bfp8._scale_bytes(*kmj.shape, "cuda").copy_(kmj)
        return sd, kmj, "act_km"

    # A: role_n = stored [M][K] ('N'); B: role_n = stored [N][K] ('T')
    sa, sak, mak = scales(M, layout[0] == "N", ma)
    sb, sbk, mbk = scales(N, layout[1] == "T", mb)
    fn = bfp8.gemm_mx if mx else bfp8.gemm
    ref = fn(layout, qa, sa, qb, sb, ma, mb)
    got = fn(layout, qa, sak, qb, sbk, mak if ma != "block" else ma, mbk if mb != "block" else mb)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int16), got.view(torch.int16))


@pytest.mark.parametrize("shape", [(301, 270, 1024), (1, 130, 640), (259, 513, 1152)])
@pytest.mark.parametrize("mb", ["block", "act"])
@pytest.mark.parametrize("mx", [False, True])
def test_gemm_kmajor_scales_unaligned_rows(shape, mb, mx):
    """Row counts that are not multiples of 4: the K-block-major scale bytes
    of a tile then start at a different offset within a word in every K
    block (the power-of-two kernel stages them as bytes from the aligned
    word before the first)."""
    M, N, K = shape
    KB = K // 128
    g = torch.Generator(device="cuda").manual_seed(M + N + K)
    qa, qb = codes((M, K), g), codes((N, K), g)

    def act_scales(rows):
        if mx:
            s = torch.randint(118, 137, (rows, KB), dtype=torch.uint8, device="cuda", generator=g)
            return bfp8._scale_bytes(rows, KB, "cuda").copy_(s), \
                bfp8._scale_bytes(KB, rows, "cuda").copy_(s.t())
        s = (torch.rand((rows, KB), device="cuda", generator=g) + 0.5).contiguous()
        return s, s.t().contiguous()

    sa, sak = act_scales(M)
    if mb == "block":
        shp = ((N + 127) // 128, KB)
        sb = (bfp8._scale_bytes(*shp, "cuda").copy_(
            torch.randint(118, 137, shp, dtype=torch.uint8, device="cuda", generator=g)) if mx
              else (torch.rand(shp, device="cuda", generator=g) + 0.5).contiguous())
        sbk, mbk = sb, "block"
    else:
        sb, sbk = act_scales(N)
        mbk = "act_km"
    fn = bfp8.gemm_mx if mx else bfp8.gemm
    ref = fn("NT", qa, sa, qb, sb, "act", mb)
    got = fn("NT", qa, sak, qb, sbk, "act_km", mbk)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int16), got.view(torch.int16))
