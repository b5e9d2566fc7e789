"""GPU parity of bfp8_gemm against the float64 oracle.

Tolerance (the bar for floating point): rel_error(C, R) <= 1e-2, where
rel_error = max|C - R| / max(|R|, rms(R)) and R is the float64 product of
the dequantised operands (oracle.gemm_ref).  The bf16 store contributes up
to 2**-9 relative; the FP8 matrix-core dot product adds its 128 products in
groups whose small terms are aligned to the largest one (about 2**-11 of the
largest product in the worst random-code case), which bounds the error of a
cancelling output relative to rms(R), not to R itself.
Integer-exact operands (codes decoding to small integers, power-of-two
scales, K <= 1024) make every fp32 step exact, so there C must equal
bf16_rne(R) bit for bit.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
import pins

pytestmark = pytest.mark.gpu

import blockwise_fp8_gemm_bfp8_amd as bfp8  # noqa: E402

TOL = 1e-2
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


def oracle_ref_ragged(layout, qa, sa, ma, qb, sb, mb, M, N):
    """gemm_ref with block-mode scale grids expanded for ragged M/N.

    For ragged extents the block grid has ceil(extent/128) entries; padding
    the stored operands to a multiple of 128 (zero codes) and cropping the
    result is the same product."""
    def pad(q, s, role, mode):
        trans = layout[0] if role == "A" else layout[1]
        mn_axis = (0 if trans == "N" else 1) if role == "A" else (1 if trans == "N" else 0)
        ext = q.shape[mn_axis]
        padded = -(-ext // 128) * 128
        if padded == ext:
            return q, s
        pw = [(0, 0), (0, 0)]
        pw[mn_axis] = (0, padded - ext)
        q = np.pad(q, pw)
        if mode == "act":
            s = np.pad(s, pw, constant_values=1.0)
        return q, s
    qa2, sa2 = pad(qa, sa, "A", ma)
    qb2, sb2 = pad(qb, sb, "B", mb)
    R = oracle.gemm_ref(layout, qa2, sa2, ma, qb2, sb2, mb)
    return R[:M, :N]


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
    R = oracle_ref_ragged(layout, qa, sa, ma, qb, sb, mb, M, N)
    C, _ = run_gpu(layout, qa, sa, ma, qb, sb, mb)
    err = oracle.rel_error(C, R)
    assert err <= TOL, (layout, modes, M, N, K, err)


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
    R = oracle_ref_ragged("NT", qa, sa, "act", qb, sb, "block", M, N)
    assert oracle.rel_error(big[:, :N].float().cpu().numpy(), R) <= TOL
    assert (big[:, N:] == 3.0).all()


def test_gemm_deterministic():
    rng = np.random.default_rng(5)
    qa, sa, qb, sb = random_operands(rng, "NT", 1024, 1024, 2048, "act", "act")
    _, c1 = run_gpu("NT", qa, sa, "act", qb, sb, "act")
    _, c2 = run_gpu("NT", qa, sa, "act", qb, sb, "act")
    assert torch.equal(c1, c2)


def test_matrix_core_alignment_loss():
    """Documents the FP8 matrix-core summation behind the tolerance reading.

    One 128-deep block, unit scales: row 0 of A is [448, 448, 1, ..., 1] and
    column 0 of B is [448, -448, 1, ..., 1], so the exact result is 126.  The
    matrix core adds products in groups of 8 aligned to the group's largest
    term, so the six 1*1 products sharing a group with the cancelling pair are
    lost (120 on gfx950).  The error stays tiny next to the largest product,
    which is what the rms-floored relative error bounds."""
    M = N = 128
    K = 128
    qa = np.zeros((M, K), np.uint8)
    qb = np.zeros((N, K), np.uint8)   # B 'T': [N][K]
    qa[0, :] = 0x38                   # 1.0
    qb[0, :] = 0x38
    qa[0, 0] = qa[0, 1] = 0x7E        # 448
    qb[0, 0], qb[0, 1] = 0x7E, 0xFE   # 448, -448
    sa = np.ones((M, 1), np.float32)
    sb = np.ones((1, 1), np.float32)
    C, _ = run_gpu("NT", qa, sa, "act", qb, sb, "block")
    exact = 126.0
    got = C[0, 0]
    assert 0.0 <= got <= exact
    assert abs(got - exact) <= 2.0 ** -11 * 448.0 * 448.0
    print(f"matrix-core result {got} for exact {exact}")


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
    R = oracle_ref_ragged("NT", qa, sa, ma, qb, sb, mb, M, N)
    t = dev_padded
    args = (t(qa), dense(sa), t(qb), dense(sb), ma, mb)
    split = bfp8.gemm("NT", *args)
    unsplit = bfp8.gemm("NT", *args, split_k=False)
    again = bfp8.gemm("NT", *args)
    torch.cuda.synchronize()
    assert oracle.rel_error(split.float().cpu().numpy(), R) <= TOL
    assert oracle.rel_error(unsplit.float().cpu().numpy(), R) <= TOL
    assert torch.equal(split, again)  # deterministic reduction order
