"""GPU parity of the power-of-two (E8M0) path against the CPU oracle (oracle/mx.py).

Quantisers: bit-exact codes and bit-exact scale bytes, groups of 32 and 128.
GEMM: the gate of tests/gate.py (|C - R| <= 1e-2 |R| + (1 + 2**-9) E, E from
the matrix core's pinned arithmetic; the scaled MFMA sums its groups of 8 the
same way, tests/test_mfma_arithmetic.py) against the float64 product of the
dequantised operands, and bit-exact bf16 where every fp32 step is exact
(integer-valued codes).
"""
import itertools

import numpy as np
import pytest
import torch

import gate
import oracle
import pins_mx
from workloads import make_inputs, to_numpy_input

pytestmark = pytest.mark.gpu

import blockwise_fp8_gemm_bfp8_amd as bfp8  # noqa: E402


def dev(t):
    """Device copy whose rows start 16-byte aligned (padded leading dim)."""
    if isinstance(t, np.ndarray):
        t = torch.from_numpy(np.ascontiguousarray(t))
    R, C = t.shape
    per = 16 // t.element_size()
    ld = max(-(-C // per) * per, per)
    buf = torch.zeros((R, ld), dtype=t.dtype, device="cuda")
    buf[:, :C] = t.to("cuda")
    return buf[:, :C]


def scales_dev(s):
    """Dense uint8 scale tensor with 4 readable bytes past its end."""
    s = np.ascontiguousarray(s, dtype=np.uint8)
    buf = torch.zeros((s.size + 4,), dtype=torch.uint8, device="cuda")
    buf[:s.size] = torch.from_numpy(s.reshape(-1)).cuda()
    return buf[:s.size].view(*s.shape)


def same(got_q, got_s, exp_q, exp_s, what=""):
    gq, gs = got_q.cpu().numpy(), got_s.cpu().numpy()
    bad = np.argwhere(gq != exp_q)
    assert bad.size == 0, f"{what}: {len(bad)} byte mismatches, first {bad[:5].tolist()}"
    assert gs.shape == exp_s.shape, (gs.shape, exp_s.shape)
    bad = np.argwhere(gs != exp_s)
    assert bad.size == 0, f"{what}: {len(bad)} scale mismatches, first {bad[:5].tolist()}"


def rand(shape, seed, dtype, std=1.0, heavy=False):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(shape, generator=g) * std
    if heavy:
        x = x * torch.exp(torch.randn(shape, generator=g) * 2)
    return x.to(dtype)


def boundary_groups(group):
    """Groups whose amax sits on / next to 448 * 2**k (where the exponent
    steps), plus zero, signed-zero, tiny and huge groups."""
    rows = []
    rng = np.random.default_rng(group)
    for k in (-100, -20, -7, -1, 0, 1, 9, 60, 110):
        base = np.float32(448.0 * 2.0 ** k)
        for amax in (base, np.nextafter(base, np.float32(np.inf)), np.nextafter(base, np.float32(0)),
                     np.float32(base * 0.5), np.float32(base * 0.75)):
            r = (rng.uniform(-1, 1, group) * amax).astype(np.float32)
            r[int(rng.integers(group))] = -amax
            rows.append(r)
    rows.append(np.zeros(group, np.float32))
    z = np.zeros(group, np.float32); z[::2] = -0.0; rows.append(z)
    rows.append((np.linspace(-1, 1, group) * 3e38).astype(np.float32))
    return np.concatenate(rows).reshape(-1, 128).astype(np.float32)


# ---------------------------------------------------------------- quantisers


@pytest.mark.parametrize("group", [32, 128])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rows,cols", [(1, 128), (3, 384), (777, 2048), (256, 6144)])
def test_mx_act(group, dtype, rows, cols):
    x = rand((rows, cols), rows * 3 + cols + group, dtype, 2.0, heavy=True)
    q, s = bfp8.quantize_mx_act(dev(x), group)
    eq, es = oracle.quantize_mx_act(to_numpy_input(x), group)
    same(q, s, eq, es, f"mx act {group} {rows}x{cols} {dtype}")


@pytest.mark.parametrize("group", [32, 128])
def test_mx_act_exponent_boundaries(group):
    x = boundary_groups(group)
    q, s = bfp8.quantize_mx_act(torch.from_numpy(x).cuda(), group)
    eq, es = oracle.quantize_mx_act(x, group)
    same(q, s, eq, es, f"boundaries {group}")


@pytest.mark.parametrize("group", [32, 128])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rows,cols", [(128, 1), (128, 100), (384, 384), (1024, 2100)])
def test_mx_act_transposed(group, dtype, rows, cols):
    x = rand((rows, cols), rows + cols * 5 + group, dtype, 0.5, heavy=True)
    qt, st = bfp8.quantize_mx_act_transposed(dev(x), group)
    eq, es = oracle.quantize_mx_act_transposed(to_numpy_input(x), group)
    same(qt, st, eq, es, f"mx transposed {group} {rows}x{cols}")


@pytest.mark.parametrize("group", [32, 128])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rows,cols", [(128, 128), (384, 256), (1024, 2048), (256, 6144)])
def test_mx_act_dual(group, dtype, rows, cols):
    # 6144 channels: the 128 x 256 tile form for bf16
    x = rand((rows, cols), rows * 11 + cols + group, dtype, 1.0, heavy=True)
    q, s, qt, st = bfp8.quantize_mx_act_dual(dev(x), group)
    xn = to_numpy_input(x)
    eq, es = oracle.quantize_mx_act(xn, group)
    eqt, est = oracle.quantize_mx_act_transposed(xn, group)
    same(q, s, eq, es, "dual rows")
    same(qt, st, eqt, est, "dual tokens")


def test_mx_dual_boundaries():
    b = boundary_groups(32)                       # [n][128] rows of boundary groups
    x = np.ascontiguousarray(np.tile(b, (-(-128 // b.shape[0]), 2))[:128])  # [128][256]
    x[:, 128:] = x[::-1, 128:].copy()             # different token groups in the right half
    for group in (32, 128):
        q, s, qt, st = bfp8.quantize_mx_act_dual(torch.from_numpy(x).cuda(), group)
        eq, es = oracle.quantize_mx_act(x, group)
        eqt, est = oracle.quantize_mx_act_transposed(x, group)
        same(q, s, eq, es, f"dual boundary rows {group}")
        same(qt, st, eqt, est, f"dual boundary tokens {group}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rows,cols", [(128, 128), (300, 200), (2048, 6144)])
def test_mx_weight(dtype, rows, cols):
    w = rand((rows, cols), rows + cols, dtype, 0.02, heavy=True)
    q, s = bfp8.quantize_mx_weight(dev(w))
    eq, es = oracle.quantize_mx_weight(to_numpy_input(w))
    same(q, s, eq, es, f"mx weight {rows}x{cols}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_mx_weight_batch_matches_oracle_and_single_calls(dtype):
    """One launch over weights of mixed sizes (ragged edge blocks, an empty
    weight): each job's codes and scale bytes equal the oracle's and the
    single call's."""
    shapes = [(128, 128), (300, 200), (0, 128), (2048, 6144), (2048, 2048)]
    ws = [rand((r, c), 7 * i + r + c, dtype, 0.02, heavy=True) for i, (r, c) in enumerate(shapes)]
    got = bfp8.quantize_mx_weight_batch([dev(w) for w in ws])
    for (r, c), w, (q, s) in zip(shapes, ws, got):
        if r == 0:
            continue
        eq, es = oracle.quantize_mx_weight(to_numpy_input(w))
        same(q, s, eq, es, f"mx weight batch {r}x{c}")
        q1, s1 = bfp8.quantize_mx_weight(dev(w))
        assert torch.equal(q, q1) and torch.equal(s, s1)


# ---------------------------------------------------------------- GEMM


def run_mx(layout, qa, sa, ma, qb, sb, mb, **kw):
    C = bfp8.gemm_mx(layout, dev(qa), scales_dev(sa), dev(qb), scales_dev(sb), ma, mb, **kw)
    torch.cuda.synchronize()
    return C


def ref_mx(layout, qa, sa, ma, qb, sb, mb):
    return oracle.gemm_mx_ref(layout, qa, sa, ma, qb, sb, mb)


MX_CASES = [("NT", "act", "block"), ("NT", "act", "act"), ("NT", "mx32", "mx32"),
            ("NT", "mx32", "block"), ("NT", "block", "mx32"), ("NT", "block", "block"),
            ("NN", "act", "block"), ("NN", "mx32", "block"), ("NN", "act", "act"),
            ("TN", "act", "act"), ("TN", "block", "block")]


@pytest.mark.parametrize("layout,ma,mb", MX_CASES)
@pytest.mark.parametrize("M,N,K", [(256, 256, 128), (300, 520, 640), (513, 129, 384)])
def test_gemm_mx_random(layout, ma, mb, M, N, K):
    rng = np.random.default_rng(M + 3 * N + 7 * K + len(ma) * 13 + len(mb))
    qa, sa, qb, sb = pins_mx.random_mx_operands(rng, layout, ma, mb, M, N, K)
    C = run_mx(layout, qa, sa, ma, qb, sb, mb)
    gate.check_stored(C.float().cpu().numpy(), layout, qa, sa, ma, qb, sb, mb,
                      (layout, ma, mb, M, N, K), mx=True)


def integer_mx_operands(rng, layout, ma, mb, M, N, K):
    """Codes decoding to integers in [-8, 8] and E8M0 scales in 2**[-2, 2]."""
    qa, sa, qb, sb = pins_mx.random_mx_operands(rng, layout, ma, mb, M, N, K)
    dec = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    ints = np.array([c for c in range(256) if np.isfinite(dec[c]) and float(dec[c]).is_integer()
                     and abs(dec[c]) <= 8], np.uint8)
    qa = rng.choice(ints, qa.shape).astype(np.uint8)
    qb = rng.choice(ints, qb.shape).astype(np.uint8)
    sa = rng.integers(125, 130, sa.shape).astype(np.uint8)
    sb = rng.integers(125, 130, sb.shape).astype(np.uint8)
    return qa, sa, qb, sb


@pytest.mark.parametrize("layout,ma,mb", MX_CASES)
def test_gemm_mx_integer_exact_bitwise(layout, ma, mb):
    rng = np.random.default_rng(21)
    M, N, K = 512, 384, 512
    qa, sa, qb, sb = integer_mx_operands(rng, layout, ma, mb, M, N, K)
    R = ref_mx(layout, qa, sa, ma, qb, sb, mb)
    exp = torch.from_numpy(R).float().to(torch.bfloat16)
    got = run_mx(layout, qa, sa, ma, qb, sb, mb).cpu()
    bad = (got.view(torch.int16) != exp.view(torch.int16)).nonzero()
    assert bad.numel() == 0, (layout, ma, mb, bad[:5].tolist())


@pytest.mark.parametrize("layout,ma,mb", [("NT", "act", "block"), ("NN", "act", "block"),
                                          ("TN", "act", "act"), ("NT", "mx32", "mx32")])
@pytest.mark.parametrize("K", [384, 512])
def test_gemm_mx_persistent_tiles_bitwise(layout, ma, mb, K):
    """More 256x256 tiles than workgroups (272 for 256 CUs), so a workgroup
    runs a second tile whose first K block its first tile's last block
    copied; the second tiles include the ragged last row and column of
    tiles; an odd K-block count (384) starts the second tile in the other
    LDS stage.  Integer-valued codes and power-of-two scales make every fp32
    step exact, so the bf16 output must match the float64 product bit for
    bit."""
    rng = np.random.default_rng(K + len(layout) + 5 * len(ma))
    M, N = 16 * 256 + 4, 15 * 256 + 200
    qa, sa, qb, sb = integer_mx_operands(rng, layout, ma, mb, M, N, K)
    R = ref_mx(layout, qa, sa, ma, qb, sb, mb)
    exp = torch.from_numpy(R).float().to(torch.bfloat16)
    got = run_mx(layout, qa, sa, ma, qb, sb, mb).cpu()
    bad = (got.view(torch.int16) != exp.view(torch.int16)).nonzero()
    assert bad.numel() == 0, (layout, ma, mb, K, bad[:5].tolist())


@pytest.mark.parametrize("M,N,K,ma,mb", [(512, 256, 16384, "act", "act"),
                                         (2048, 2048, 16384, "mx32", "mx32")])
def test_gemm_mx_split_k(M, N, K, ma, mb):
    rng = np.random.default_rng(M + N)
    qa, sa, qb, sb = pins_mx.random_mx_operands(rng, "NT", ma, mb, M, N, K)
    assert bfp8.gemm_workspace_bytes("NT", ma, mb, M, N, K) > 0
    parts = gate.operand_parts("NT", qa, sa, ma, qb, sb, mb, mx=True)
    R = gate.reference(*parts)
    split = run_mx("NT", qa, sa, ma, qb, sb, mb)
    unsplit = run_mx("NT", qa, sa, ma, qb, sb, mb, split_k=False)
    gate.check(split.float().cpu().numpy(), *parts, ("split", M, N, K), R=R)
    gate.check(unsplit.float().cpu().numpy(), *parts, ("unsplit", M, N, K), R=R)


@pytest.mark.parametrize("group", [32, 128])
def test_mx_linear_layer_end_to_end(group):
    """fprop / dgrad / wgrad of one linear with power-of-two scales, from
    bf16 inputs through the MX quantisers and gemm_mx, against the oracle
    run on the same inputs (sampled rows of a 2048-token batch)."""
    t = make_inputs("qkv_fprop_m8192")
    x = t["x.qkv"][:2048]
    w = t["w.qkv"][:1024]
    dy = rand((2048, 1024), 99, torch.bfloat16, 1e-3)
    xn, wn, dyn = to_numpy_input(x), to_numpy_input(w), to_numpy_input(dy)
    mode = "mx32" if group == 32 else "act"
    # GPU
    xq, xs, xqt, xst = bfp8.quantize_mx_act_dual(dev(x), group)
    dq, ds, dqt, dst = bfp8.quantize_mx_act_dual(dev(dy), group)
    if group == 32:
        wq, ws, wqt, wst = bfp8.quantize_mx_act_dual(dev(w), 32)
        y = bfp8.gemm_mx("NT", xq, xs, wq, ws, mode, mode)
        dx = bfp8.gemm_mx("NT", dq, ds, wqt, wst, mode, mode)
    else:
        wq, ws = bfp8.quantize_mx_weight(dev(w))
        y = bfp8.gemm_mx("NT", xq, xs, wq, ws, mode, "block")
        dx = bfp8.gemm_mx("NN", dq, ds, wq, ws, mode, "block")
    dw = bfp8.gemm_mx("NT", dqt, dst, xqt, xst, mode, mode)
    torch.cuda.synchronize()
    # oracle, on sampled rows / all of dW
    rows = np.arange(0, 2048, 97)
    eq, es = oracle.quantize_mx_act(xn[rows], group)
    dqo, dso = oracle.quantize_mx_act(dyn[rows], group)
    if group == 32:
        wqo, wso = oracle.quantize_mx_act(wn, 32)
        wqto, wsto = oracle.quantize_mx_act_transposed(wn, 32)
        py = gate.operand_parts("NT", eq, es, mode, wqo, wso, mode, mx=True)
        pdx = gate.operand_parts("NT", dqo, dso, mode, wqto, wsto, mode, mx=True)
    else:
        wqo, wso = oracle.quantize_mx_weight(wn)
        py = gate.operand_parts("NT", eq, es, mode, wqo, wso, "block", mx=True)
        pdx = gate.operand_parts("NN", dqo, dso, mode, wqo, wso, "block", mx=True)
    xqto, xsto = oracle.quantize_mx_act_transposed(xn, group)
    dqto, dsto = oracle.quantize_mx_act_transposed(dyn, group)
    pdw = gate.operand_parts("NT", dqto, dsto, mode, xqto, xsto, mode, mx=True)
    gate.check(y.float().cpu().numpy()[rows], *py, ("mx fprop", group))
    gate.check(dx.float().cpu().numpy()[rows], *pdx, ("mx dgrad", group))
    gate.check(dw.float().cpu().numpy(), *pdw, ("mx wgrad", group))


def test_gemm_mx_hybrid_split_plan():
    """33 x 8 tiles at K = 4096 on the persistent power-of-two kernel: 256
    whole tiles in one launch, then the last row of 8 tiles split along K in
    a second launch that starts 8192 rows into A, its scales and C.  The
    whole tiles equal the unsplit plan's bytes (a plan that split every tile
    would sum them in another order); sampled rows, every split row
    included, meet the parity bound.  K-block-major A scales are copied,
    rows 8192.. of every K block, before the second launch."""
    M, N, K = 8448, 2048, 4096
    rng = np.random.default_rng(23)
    rows = np.r_[0:8192:61, 8192:M]
    for layout, ma, mb in (("NT", "act", "act"), ("NT", "mx32", "mx32"), ("NT", "act", "block"),
                           ("TN", "act", "act"), ("NT", "act_km", "act_km")):
        base = (ma.replace("_km", ""), mb.replace("_km", ""))
        qa, sa, qb, sb = pins_mx.random_mx_operands(rng, layout, *base, M, N, K)
        if ma == "act_km":  # K-block-major scale bytes, [K/128][rows]
            sa_r, sb_r = sa, sb
            sa, sb = np.ascontiguousarray(sa.T), np.ascontiguousarray(sb.T)
        assert bfp8.gemm_workspace_bytes(layout, ma, mb, M, N, K) > 0  # a split plan
        hybrid = run_mx(layout, qa, sa, ma, qb, sb, mb)
        unsplit = run_mx(layout, qa, sa, ma, qb, sb, mb, split_k=False)
        again = run_mx(layout, qa, sa, ma, qb, sb, mb)
        assert torch.equal(hybrid, again)
        assert torch.equal(hybrid[:8192].view(torch.int16), unsplit[:8192].view(torch.int16))
        # A's sampled rows: stored rows for 'N', stored columns for 'T' (1x128 scales)
        if ma == "act_km":
            parts = gate.operand_parts(layout, qa[rows], sa_r[rows], "act", qb, sb_r, "act", mx=True)
        else:
            qs, ss = (qa[rows], sa[rows]) if layout[0] == "N" else (qa[:, rows], sa[:, rows])
            parts = gate.operand_parts(layout, qs, ss, ma, qb, sb, mb, mx=True)
        for name, C in (("hybrid", hybrid), ("unsplit", unsplit)):
            gate.check(C.float().cpu().numpy()[rows], *parts, (name, layout, ma, mb), mx=True)
