"""GPU parity of bfp8_gemm against the float64 oracle.

The bar for floating point (tests/gate.py, oracle/tolerance.py): every output
satisfies |C - R| <= 1e-2 |R| + (1 + 2**-9) E, where R is the float64 product
of the dequantised operands (oracle.gemm_ref) and E bounds the error of the
matrix core's measured arithmetic (groups of 8 products truncated to 13 bits
below their largest exponent sum, float32 sums; pinned exactly by
tests/test_mfma_arithmetic.py).  The survey's O6 figure is printed beside it.
Integer-exact operands (codes decoding to small integers, power-of-two
scales, K <= 1024) make every fp32 step exact, so there C must equal
bf16_rne(R) bit for bit.
"""
import itertools

import numpy as np
import pytest
import torch

import gate
import oracle
import pins

pytestmark = pytest.mark.gpu

import blockwise_fp8_gemm_bfp8_amd as bfp8  # noqa: E402

LAYOUTS = ["NT", "NN", "TN"]
MODES = [("act", "block"), ("act", "act"), ("block", "act"), ("block", "block")]


def stored_shapes(layout, M, N, K, ma, mb):
    """Stored byte and scale shapes of A and B for a layout and modes."""
    cd = lambda a: (a + 127) // 128
    a_shape = (M, K) if layout[0] == "N" else (K, M)
    b_shape = (K, N) if layout[1] == "N" else (N, K)
    if ma == "act":
        sa = (M, K // 128) if layout[0] == "N" else (K // 128, M)
    else:
        sa = (cd(M), K // 128) if layout[0] == "N" else (K // 128, cd(M))
    if mb == "act":
        sb = (K // 128, N) if layout[1] == "N" else (N, K // 128)
    else:
        sb = (K // 128, cd(N)) if layout[1] == "N" else (cd(N), K // 128)
    return a_shape, sa, b_shape, sb


def random_operands(rng, layout, M, N, K, ma, mb):
    a_shape, sa_shape, b_shape, sb_shape = stored_shapes(layout, M, N, K, ma, mb)
    qa = rng.integers(0, 256, a_shape).astype(np.uint8)
    qb = rng.integers(0, 256, b_shape).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x7E  # no NaN codes
    qb[(qb & 0x7F) == 0x7F] = 0x7E
    sa = (rng.uniform(0.5, 2.0, sa_shape) * 2.0 ** rng.integers(-8, 8, sa_shape)).astype(np.float32)
    sb = (rng.uniform(0.5, 2.0, sb_shape) * 2.0 ** rng.integers(-8, 8, sb_shape)).astype(np.float32)
    return qa, sa, qb, sb


def dev_padded(a):
    """Device copy of a 2-D array whose rows start 16-byte aligned."""
    a = np.ascontiguousarray(a)
    if a.ndim != 2:
        return torch.from_numpy(a).cuda()
    R, C = a.shape
    per = 16 // a.itemsize
    ld = max(-(-C // per) * per, per)
    buf = torch.zeros((R, ld), dtype=torch.from_numpy(a[:0]).dtype, device="cuda")
    buf[:, :C] = torch.from_numpy(a).cuda()
    return buf[:, :C]


def dense(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_gpu(layout, qa, sa, ma, qb, sb, mb):
    t = dev_padded  # codes: padded leading dimension; scales: dense
    C = bfp8.gemm(layout, t(qa), dense(sa), t(qb), dense(sb), ma, mb)
    torch.cuda.synchronize()
    return C.float().cpu().numpy().astype(np.float64), C


@pytest.mark.parametrize("layout,modes", list(itertools.product(LAYOUTS, MODES)))
@pytest.mark.parametrize("M,N,K", [(256, 256, 128), (300, 520, 640), (513, 129, 384)])
def test_random_codes_within_tolerance(layout, modes, M, N, K):
    rng = np.random.default_rng(M * 31 + N * 7 + K)
    ma, mb = modes
    qa, sa, qb, sb = random_operands(rng, layout, M, N, K, ma, mb)
    C, _ = run_gpu(layout, qa, sa, ma, qb, sb, mb)
    gate.check_stored(C, layout, qa, sa, ma, qb, sb, mb, (layout, modes, M, N, K))


@pytest.mark.parametrize("layout,modes", list(itertools.product(LAYOUTS, MODES)))
def test_integer_exact_bitwise(layout, modes):
    rng = np.random.default_rng(11)
    ma, mb = modes
    M, N, K = 512, 384, 1024
    qa, sa, qb, sb = pins.integer_exact_operands(rng, layout, ma, mb, M, N, K)
    R = oracle.gemm_ref(layout, qa, sa, ma, qb, sb, mb)
    exp = torch.from_numpy(R).float().to(torch.bfloat16)  # library RNE of the exact sum
    _, Cd = run_gpu(layout, qa, sa, ma, qb, sb, mb)
    got = Cd.cpu()
    bad = (got.view(torch.int16) != exp.view(torch.int16)).nonzero()
    assert bad.numel() == 0, (layout, modes, bad[:5].tolist())


def test_k_zero_writes_zeros_and_empty_is_noop():
    C = torch.full((64, 80), 7.0, dtype=torch.bfloat16, device="cuda")
    qa = torch.zeros((64, 0), dtype=torch.uint8, device="cuda")
    qb = torch.zeros((80, 0), dtype=torch.uint8, device="cuda")
    s = torch.ones((256,), dtype=torch.float32, device="cuda")
    bfp8.gemm("NT", qa, s, qb, s, "act", "block", out=C)
    assert (C == 0).all()
    C2 = torch.full((0, 80), 7.0, dtype=torch.bfloat16, device="cuda")
    bfp8.gemm("NT", torch.zeros((0, 128), dtype=torch.uint8, device="cuda"), s,
              torch.zeros((80, 128), dtype=torch.uint8, device="cuda"), s, "act", "block", out=C2)


def test_output_leading_dimension_and_padding():
    rng = np.random.default_rng(3)
    M, N, K = 300, 200, 256
    qa, sa, qb, sb = random_operands(rng, "NT", M, N, K, "act", "block")
    t = dev_padded
    big = torch.full((M, 264), 3.0, dtype=torch.bfloat16, device="cuda")
    bfp8.gemm("NT", t(qa), dense(sa), t(qb), dense(sb), "act", "block", out=big[:, :N])
    gate.check_stored(big[:, :N].float().cpu().numpy(), "NT", qa, sa, "act", qb, sb, "block",
                      "ldc 264")
    assert (big[:, N:] == 3.0).all()


def test_gemm_deterministic():
    rng = np.random.default_rng(5)
    qa, sa, qb, sb = random_operands(rng, "NT", 1024, 1024, 2048, "act", "act")
    _, c1 = run_gpu("NT", qa, sa, "act", qb, sb, "act")
    _, c2 = run_gpu("NT", qa, sa, "act", qb, sb, "act")
    assert torch.equal(c1, c2)


@pytest.mark.parametrize("M,N,K,modes", [(512, 256, 16384, ("act", "act")),
                                         (300, 250, 8192, ("act", "block")),
                                         (2048, 2048, 16384, ("act", "act"))])
def test_split_k_matches_oracle_and_unsplit(M, N, K, modes):
    """Shapes whose tiles under-fill the GPU take the split-K plan (fp32
    partials summed in split order); both plans must meet the tolerance."""
    rng = np.random.default_rng(M + N + K)
    ma, mb = modes
    qa, sa, qb, sb = random_operands(rng, "NT", M, N, K, ma, mb)
    assert bfp8.gemm_workspace_bytes("NT", ma, mb, M, N, K) > 0
    parts = gate.operand_parts("NT", qa, sa, ma, qb, sb, mb)
    R = gate.reference(*parts)
    t = dev_padded
    args = (t(qa), dense(sa), t(qb), dense(sb), ma, mb)
    split = bfp8.gemm("NT", *args)
    unsplit = bfp8.gemm("NT", *args, split_k=False)
    again = bfp8.gemm("NT", *args)
    torch.cuda.synchronize()
    gate.check(split.float().cpu().numpy(), *parts, ("split", M, N, K), R=R)
    gate.check(unsplit.float().cpu().numpy(), *parts, ("unsplit", M, N, K), R=R)
    assert torch.equal(split, again)  # deterministic reduction order


@pytest.mark.parametrize("M,N,modes", [(8448, 2048, ("act", "act")), (8448, 2048, ("act", "block")),
                                        (8348, 2000, ("act", "act"))])
def test_hybrid_split_plan(M, N, modes):
    """A tile grid one wave and a bit (33 x 8 tiles of 256 x 256 at K = 4096,
    the last row and column of tiles ragged in the third case): the first 256
    tiles run unsplit and only the last row of 8 tiles is split along K (its
    fp32 partials, rows 8192.. only, summed in split order).  The unsplit
    tiles must equal the unsplit plan's bytes (a plan that split every tile
    would sum them in another order); every sampled row, the split rows
    included, must meet the parity bound."""
    K = 4096
    ma, mb = modes
    rng = np.random.default_rng(17 + len(mb))
    qa, sa, qb, sb = random_operands(rng, "NT", M, N, K, ma, mb)
    assert bfp8.gemm_workspace_bytes("NT", ma, mb, M, N, K) > 0  # a split plan
    t = dev_padded
    args = (t(qa), dense(sa), t(qb), dense(sb), ma, mb)
    hybrid = bfp8.gemm("NT", *args)
    unsplit = bfp8.gemm("NT", *args, split_k=False)
    again = bfp8.gemm("NT", *args)
    torch.cuda.synchronize()
    assert torch.equal(hybrid, again)  # deterministic reduction order
    assert torch.equal(hybrid[:8192].view(torch.int16), unsplit[:8192].view(torch.int16))
    rows = np.r_[0:8192:61, 8192:M]
    bc, bsc = oracle.logical_operand(qb, sb, "B", "T", mb)
    ac, asc = oracle.logical_operand(qa[rows], sa[rows], "A", "N", ma)  # 1x128 A scales
    for name, C in (("hybrid", hybrid), ("unsplit", unsplit)):
        gate.check(C.float().cpu().numpy()[rows], ac, asc, bc, bsc, (name, M, N, K, modes))


@pytest.mark.parametrize("M,modes", [(2048, ("act", "act")), (2000, ("act", "act")),
                                     (2048, ("act_km", "act_km")), (2048, ("act", "act_km"))])
def test_192_column_tiles(M, modes):
    """An NT GEMM with 1x128 scales on B and N = 6144 (the 2048 x 6144 wgrad
    output) runs as 256 x 192 tiles, 8 x 32 of them, where 256-column tiles
    would leave 64 CUs idle.  Every output is summed in the same order as
    with 256-column tiles, so the bytes must equal those of N = 6152 (which
    does not divide by 192 and runs 256-column tiles) on the shared columns;
    sampled rows, the ragged last row tile included, meet the parity bound."""
    N, K = 6144, 2048
    ma, mb = modes
    rng = np.random.default_rng(M + len(ma) + 3 * len(mb))
    base = [m.replace("_km", "") for m in modes]
    qa, sa, qb, sb = random_operands(rng, "NT", M, N + 8, K, *base)
    sa_d = dense(sa) if ma == "act" else dense(np.ascontiguousarray(sa.T))   # [K/128][M]
    sbk = sb if mb == "act" else np.ascontiguousarray(sb.T)                  # [K/128][N]
    narrow = bfp8.gemm("NT", dev_padded(qa), sa_d, dev_padded(qb[:N]),
                       dense(sbk[:N] if mb == "act" else sbk[:, :N]), ma, mb)
    wide = bfp8.gemm("NT", dev_padded(qa), sa_d, dev_padded(qb), dense(sbk), ma, mb)
    torch.cuda.synchronize()
    assert torch.equal(narrow.view(torch.int16), wide[:, :N].view(torch.int16))
    rows = np.r_[0:M:37, M - 16:M]
    ac, asc = oracle.logical_operand(qa[rows], sa[rows], "A", "N", "act")
    bc, bsc = oracle.logical_operand(qb[:N], sb[:N], "B", "T", "act")
    gate.check(narrow.float().cpu().numpy()[rows], ac, asc, bc, bsc, ("192 columns", M, modes))
