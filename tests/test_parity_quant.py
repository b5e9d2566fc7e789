"""GPU parity of the three quantisers against the CPU oracle: bit-exact bytes
and bit-exact float32 scales, through the C ABI (via the thin binding)."""
import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS, make_inputs, to_numpy_input

pytestmark = pytest.mark.gpu

import blockwise_fp8_gemm_bfp8_amd as bfp8  # noqa: E402


def dev(t):
    """Device copy whose rows start 16-byte aligned (padded leading dim)."""
    if t.dim() != 2:
        return t.to("cuda")
    R, C = t.shape
    per = 16 // t.element_size()
    ld = max(-(-C // per) * per, per)
    buf = torch.zeros((R, ld), dtype=t.dtype, device="cuda")
    buf[:, :C] = t.to("cuda")
    return buf[:, :C]


def assert_same_codes(got_q, got_s, exp_q, exp_s, what=""):
    gq = got_q.cpu().numpy()
    gs = got_s.cpu().numpy()
    bad = np.argwhere(gq != exp_q)
    assert bad.size == 0, f"{what}: {len(bad)} byte mismatches, first {bad[:5].tolist()}"
    assert gs.shape == exp_s.shape
    bad = np.argwhere(gs.view(np.uint32) != exp_s.view(np.uint32))
    assert bad.size == 0, f"{what}: {len(bad)} scale mismatches, first {bad[:5].tolist()}"


def rand_bf16(shape, seed, std=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * std).to(torch.bfloat16)


# ---------------------------------------------------------------- act


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rows,cols", [(1, 128), (3, 384), (256, 512), (1000, 2048), (777, 6144)])
def test_quantize_act_shapes(dtype, rows, cols):
    g = torch.Generator().manual_seed(rows * 7 + cols)
    x = (torch.randn((rows, cols), generator=g) * 3).to(dtype)
    q, s = bfp8.quantize_act(dev(x))
    eq, es = oracle.quantize_act(to_numpy_input(x))
    assert_same_codes(q, s, eq, es, f"act {rows}x{cols} {dtype}")


def test_quantize_act_tiny_workload_fp32():
    t = make_inputs("tiny_256x512x384")
    q, s = bfp8.quantize_act(dev(t["x.tiny"]))
    eq, es = oracle.quantize_act(to_numpy_input(t["x.tiny"]))
    assert_same_codes(q, s, eq, es, "tiny X")


def test_quantize_act_strided_rows():
    # ldx > cols and ldq > cols; the padding of q must stay untouched
    big = rand_bf16((64, 1024), 5)
    q = torch.full((64, 640), 0xAB, dtype=torch.uint8, device="cuda")
    s_ = torch.empty((64, 4), dtype=torch.float32, device="cuda")
    bfp8.quantize_act(dev(big)[:, :512], q[:, :512], s_)
    eq, es = oracle.quantize_act(to_numpy_input(big[:, :512].contiguous()))
    assert_same_codes(q[:, :512], s_, eq, es, "strided")
    assert (q[:, 512:].cpu() == 0xAB).all()


def adversarial_groups():
    """Rows of 128 values that hit the corner cases of the scale and the cast."""
    rows = []
    z = np.zeros(128, np.float32)
    rows.append(z.copy())                                   # all zero
    nz = z.copy(); nz[::2] = -0.0; rows.append(nz)          # signed zeros
    sp = z.copy(); sp[17] = 3.5; rows.append(sp)            # single spike
    sp2 = z.copy(); sp2[100] = -1e-20; rows.append(sp2)     # tiny negative spike
    # amax = 448 -> inv = 1: the other values are cast as they are, so put
    # them on exact E4M3 midpoints (ties) and their neighbours
    dec = oracle.e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = ((dec[:-1] + dec[1:]) / 2).astype(np.float32)
    for off in range(0, len(mids), 127):
        r = np.full(128, 0.0, np.float32)
        chunk = mids[off:off + 127]
        r[:len(chunk)] = chunk * np.where(np.arange(len(chunk)) % 2, -1, 1)
        r[127] = 448.0
        rows.append(r)
        rows.append(np.where(r == 448.0, r, np.nextafter(r, np.float32(np.inf))).astype(np.float32))
        rows.append(np.where(r == 448.0, r, np.nextafter(r, np.float32(-np.inf))).astype(np.float32))
    # values that land just under/over 448 after scaling and the 464 tie
    r = np.linspace(-500, 500, 128).astype(np.float32); rows.append(r)
    r = np.full(128, 464.0, np.float32); r[0] = -464.0; rows.append(r)
    # huge and tiny (in-contract) magnitudes
    rows.append((np.linspace(-1, 1, 128) * 3e38).astype(np.float32))
    rows.append((np.linspace(-1, 1, 128) * np.float32(448 * 2.0 ** -126) * 1.5).astype(np.float32))
    # fp32 subnormal inputs inside a group with a normal amax
    r = np.full(128, np.float32(1e-40), np.float32); r[5] = 1e-35; r[6] = -3e-41; rows.append(r)
    return np.stack(rows).astype(np.float32)


def test_quantize_act_adversarial_fp32():
    x = adversarial_groups()
    q, s = bfp8.quantize_act(torch.from_numpy(x).cuda())
    eq, es = oracle.quantize_act(x)
    assert_same_codes(q, s, eq, es, "adversarial fp32")


def test_quantize_act_adversarial_bf16():
    x = torch.from_numpy(adversarial_groups()).to(torch.bfloat16)
    q, s = bfp8.quantize_act(dev(x))
    eq, es = oracle.quantize_act(to_numpy_input(x))
    assert_same_codes(q, s, eq, es, "adversarial bf16")


def test_cast_exhaustive_through_quantiser():
    """Every float32 in [2**-12, 2**9) of both signs, cast with inv == 1.

    Each group holds 127 test values plus +448, so amax = 448, s = 1 and
    the codes are the plain saturating RNE cast of the values."""
    rng = np.random.default_rng(0)
    for ef in range(115, 136):  # biased exponents 2**-12 .. 2**8
        bits = np.arange(1 << 23, dtype=np.uint32) | np.uint32(ef << 23)
        vals = bits.view(np.float32) * np.where(rng.random(1 << 23) < 0.5, -1, 1).astype(np.float32)
        n = (len(vals) + 126) // 127
        buf = np.zeros((n, 128), np.float32)
        flat = buf[:, :127].reshape(-1)
        flat[:len(vals)] = vals
        buf[:, :127] = flat.reshape(n, 127)
        buf[:, 127] = 448.0
        q, s = bfp8.quantize_act(torch.from_numpy(buf).cuda())
        eq, es = oracle.quantize_act(buf)
        assert_same_codes(q, s, eq, es, f"binade {ef}")


# ---------------------------------------------------------------- transposed


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rows,cols", [(128, 1), (128, 100), (384, 384), (1024, 2100), (8192, 64)])
def test_quantize_act_transposed_shapes(dtype, rows, cols):
    g = torch.Generator().manual_seed(rows + 3 * cols)
    x = (torch.randn((rows, cols), generator=g) * 2).to(dtype)
    x[:, cols // 2] = 0
    qt, st = bfp8.quantize_act_transposed(dev(x))
    eq, es = oracle.quantize_act_transposed(to_numpy_input(x))
    assert_same_codes(qt, st, eq, es, f"transposed {rows}x{cols} {dtype}")


def test_transposed_equals_act_of_transpose_on_gpu():
    x = rand_bf16((1024, 768), 9)
    qt, st = bfp8.quantize_act_transposed(dev(x))
    q2, s2 = bfp8.quantize_act(dev(x.T.contiguous()))
    assert torch.equal(qt, q2) and torch.equal(st.view(torch.int32), s2.view(torch.int32))


# ---------------------------------------------------------------- dual


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rows,cols", [(128, 128), (384, 256), (1024, 2048), (8192, 384),
                                       (256, 6144), (256, 6272), (384, 12288)])
def test_quantize_act_dual_equals_both_quantisers(dtype, rows, cols):
    # 6144 and 12288 channels take the 128 x 256 tiles for bf16 (paired
    # scale stores); 6272 = 49 blocks keeps the 128 x 128 tiles
    g = torch.Generator().manual_seed(rows * 3 + cols)
    x = (torch.randn((rows, cols), generator=g) * 2).to(dtype)
    x[:, cols // 3] = 0
    x[rows // 2, :] = 0
    q, s_, qt, st = bfp8.quantize_act_dual(dev(x))
    eq, es = oracle.quantize_act(to_numpy_input(x))
    assert_same_codes(q, s_, eq, es, f"dual rows {rows}x{cols} {dtype}")
    eqt, est = oracle.quantize_act_transposed(to_numpy_input(x))
    assert_same_codes(qt, st, eqt, est, f"dual cols {rows}x{cols} {dtype}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_quantize_act_dual_adversarial(dtype):
    # (bf16: the corner cases rounded to bf16 -- the input of the
    # code-transposing kernel that bf16 inputs under 6144 channels take)
    base = adversarial_groups()  # 12 x 128 rows of corner cases
    x = np.concatenate([base] * 11)[:128]
    x = np.concatenate([x, x.T.copy()], axis=1)  # corner cases along both axes
    xt = torch.from_numpy(np.ascontiguousarray(x)).to(dtype)
    q, s_, qt, st = bfp8.quantize_act_dual(xt.cuda())
    xn = to_numpy_input(xt)
    eq, es = oracle.quantize_act(xn)
    eqt, est = oracle.quantize_act_transposed(xn)
    assert_same_codes(q, s_, eq, es, f"dual adversarial rows {dtype}")
    assert_same_codes(qt, st, eqt, est, f"dual adversarial cols {dtype}")


# ---------------------------------------------------------------- weight


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rows,cols", [(128, 128), (384, 512), (100, 200), (300, 2048), (4096, 2048)])
def test_quantize_weight_shapes(dtype, rows, cols):
    g = torch.Generator().manual_seed(rows * 5 + cols)
    w = (torch.randn((rows, cols), generator=g) * 0.02).to(dtype)
    q, s = bfp8.quantize_weight(dev(w))
    eq, es = oracle_quantize_weight_ragged(to_numpy_input(w))
    assert_same_codes(q, s, eq, es, f"weight {rows}x{cols} {dtype}")


def oracle_quantize_weight_ragged(w):
    """Partial edge blocks: each block is quantised as one group of its valid
    elements (oracle.quantize_group); full blocks use oracle.quantize_weight."""
    w = np.asarray(w)
    if w.dtype == np.uint16:
        w = (w.astype(np.uint32) << 16).view(np.float32)
    R, C = w.shape
    if R % 128 == 0 and C % 128 == 0:
        return oracle.quantize_weight(w)
    q = np.zeros((R, C), np.uint8)
    s = np.zeros(((R + 127) // 128, (C + 127) // 128), np.float32)
    for bi in range(s.shape[0]):
        for bj in range(s.shape[1]):
            blk = w[128 * bi:128 * bi + 128, 128 * bj:128 * bj + 128]
            qb, sb = oracle.quantize_group(blk)
            q[128 * bi:128 * bi + 128, 128 * bj:128 * bj + 128] = qb
            s[bi, bj] = sb
    return q, s


def test_weight_block_with_outlier_and_zero_block():
    w = rand_bf16((256, 256), 4, 0.02)
    w[:128, :128] = 0
    w[200, 200] = 1000.0
    q, s = bfp8.quantize_weight(dev(w))
    eq, es = oracle.quantize_weight(to_numpy_input(w))
    assert_same_codes(q, s, eq, es, "weight special blocks")
    assert s[0, 0].item() == 1.0


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_quantize_weight_batch_matches_oracle_and_single_calls(dtype):
    """One launch over weights of mixed sizes (ragged edge blocks, a
    2048 x 2048 weight of 256 blocks, an empty one): each job bit-exact
    against the oracle and against bfp8_quantize_weight on it; a second
    batch on a subset into the same buffers gives the same bytes."""
    shapes = [(384, 512), (100, 200), (2048, 2048), (0, 256), (300, 2048), (128, 6144)]
    ws = []
    for i, (r, c) in enumerate(shapes):
        g = torch.Generator().manual_seed(1000 + i)
        ws.append((torch.randn((r, c), generator=g) * 0.02 * (i + 1)).to(dtype))
    got = bfp8.quantize_weight_batch([dev(w) for w in ws])
    for (r, c), w, (q, s) in zip(shapes, ws, got):
        if r == 0:
            continue
        eq, es = oracle_quantize_weight_ragged(to_numpy_input(w))
        assert_same_codes(q, s, eq, es, f"batch weight {r}x{c} {dtype}")
        q1, s1 = bfp8.quantize_weight(dev(w))
        assert torch.equal(q, q1) and torch.equal(s.view(torch.int32), s1.view(torch.int32))
    again = bfp8.quantize_weight_batch([dev(w) for w in ws[1:3]],
                                       [q for q, _ in got[1:3]], [s for _, s in got[1:3]])
    torch.cuda.synchronize()
    for (q, s), w in zip(again, ws[1:3]):
        eq, es = oracle_quantize_weight_ragged(to_numpy_input(w))
        assert_same_codes(q, s, eq, es, "batch again")


def test_quantize_weight_batch_max_jobs():
    """BFP8_MAX_WEIGHT_JOBS small weights in one launch."""
    n = bfp8.MAX_WEIGHT_JOBS
    ws = [rand_bf16((128 * (1 + i % 3), 256), 50 + i, 0.01 * (1 + i)) for i in range(n)]
    got = bfp8.quantize_weight_batch([dev(w) for w in ws])
    for w, (q, s) in zip(ws, got):
        eq, es = oracle.quantize_weight(to_numpy_input(w))
        assert_same_codes(q, s, eq, es, "max-jobs batch")


# ---------------------------------------------------------------- workloads


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_quantisers(name):
    """Every tensor of every workload: bytes and scales of all three
    quantisers (full tensors up to 8192 rows; sampled rows/channels beyond)."""
    t = make_inputs(name)
    rng = np.random.default_rng(1)
    for key, x in t.items():
        xn = to_numpy_input(x)
        xd = dev(x)
        if key.startswith("w."):
            q, s = bfp8.quantize_weight(xd)
            eq, es = oracle.quantize_weight(xn)
            assert_same_codes(q, s, eq, es, key)
            continue
        R, C = x.shape
        q, s = bfp8.quantize_act(xd)
        rows = np.arange(R) if R <= 8192 else np.sort(rng.choice(R, 512, replace=False))
        eq, es = oracle.quantize_act(xn[rows])
        assert_same_codes(q[torch.from_numpy(rows).cuda()], s[torch.from_numpy(rows).cuda()],
                          eq, es, key + " act")
        if R % 128 == 0 and ("dgrad" in WORKLOADS[name].roles or "wgrad" in WORKLOADS[name].roles):
            qt, st = bfp8.quantize_act_transposed(xd)
            cols = np.arange(C) if R * C <= 8192 * 2048 else np.sort(rng.choice(C, 96, replace=False))
            eq, es = oracle.quantize_act_transposed(np.ascontiguousarray(xn[:, cols]))
            ci = torch.from_numpy(cols).cuda()
            assert_same_codes(qt[ci], st[ci], eq, es, key + " transposed")


def test_quantisers_deterministic():
    x = dev(rand_bf16((4096, 2048), 3))
    a = bfp8.quantize_act(x)
    b = bfp8.quantize_act(x)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    a = bfp8.quantize_act_transposed(x)
    b = bfp8.quantize_act_transposed(x)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
