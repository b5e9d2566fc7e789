"""Power-of-two (E8M0) scaled E4M3 quantisers and their GEMM reference.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages say:
  * Puro-2B paper, zh-TW translation (papers.lianghsun.dev), section 3.2
    "FP8 mixed-precision training": on RTX 5090 (SM120) each logical block
    scale was constrained to a power of two and the blockwise recipe ran on
    the native MXFP8 path; the groups are unchanged (1-D groups of 128 along
    the reduction dimension for activations and activation gradients,
    128x128 blocks for weights).
  * Puro-2B tutorial (bloombook.cn), FP8/MuonH section and its MXFP figure:
    MXFP8 shares one scale X per block of 32 elements and an element decodes
    as V_i = Q_i * X.

Readings (the pages leave these open):
  * scale exponent e = the smallest integer with 448 * 2**e >= amax (the
    power of two is rounded up, so no element of the group saturates),
    clamped to [-127, 127]; an all-zero group gets e = 0;
  * code = E4M3 round-to-nearest-even of x * 2**-e (an exact scaling);
  * the scale is stored as one E8M0 byte, e + 127 (value 2**(byte - 127));
  * groups whose amax is a float32 subnormal (below 2**-126) and non-finite
    inputs are outside the contract.

The computation of e below is a search over integer candidates with exact
float64 comparisons (448 * 2**e is exact); the HIP kernels derive it from
the float32 bit fields instead.
"""

import numpy as np

from .e4m3 import e4m3_decode, e4m3_encode
from .quant import _as_f32

E8M0_BIAS = 127
_E_MIN, _E_MAX = -127, 127
MX_GROUPS = (32, 128)


def pow2_exponent(amax):
    """Smallest integer e with 448 * 2**e >= amax, clamped to [-127, 127];
    0 where amax == 0.  amax: array of non-negative float32 values."""
    a = np.asarray(amax, dtype=np.float64)
    zero = a == 0
    safe = np.where(zero, 1.0, a)
    _, E = np.frexp(safe)  # safe = m * 2**E, 0.5 <= m < 1, so 2**(E-1) <= safe < 2**E
    # 448 * 2**(E - 10) = 1.75 * 2**(E - 2) < 2**(E - 1) <= safe: a lower bound;
    # 448 * 2**(E - 8) = 1.75 * 2**E >= safe: an upper bound.  Step up to the
    # first candidate that covers amax.
    e = (E - 10).astype(np.int64)
    for _ in range(3):
        e = np.where(448.0 * np.exp2(e.astype(np.float64)) < safe, e + 1, e)
    e = np.clip(e, _E_MIN, _E_MAX)
    return np.where(zero, 0, e).astype(np.int64)


def e8m0_decode(b):
    """E8M0 byte -> float64 scale 2**(b - 127) (byte 255, NaN, is never produced)."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    return np.exp2((b - E8M0_BIAS).astype(np.float64))


def _mx_groups_last_axis(g):
    """Quantise every group g[..., :] with a power-of-two scale.

    Returns (codes uint8 of g's shape, E8M0 bytes of g.shape[:-1])."""
    g = np.asarray(g, dtype=np.float32)
    amax = np.max(np.abs(g), axis=-1).astype(np.float32)
    e = pow2_exponent(amax)
    # x * 2**-e is exact in float64; the float32 value the kernel forms is
    # the same number (no rounding: the result is at most 448)
    y = (g.astype(np.float64) * np.exp2(-e.astype(np.float64))[..., None]).astype(np.float32)
    return e4m3_encode(y), (e + E8M0_BIAS).astype(np.uint8)


def quantize_mx_group(x):
    """One group (any shape) -> (codes uint8, E8M0 scale byte)."""
    x = np.asarray(x, dtype=np.float32)
    q, b = _mx_groups_last_axis(x.reshape(1, -1))
    return q.reshape(x.shape), np.uint8(b[0])


def quantize_mx_act(x, group=128):
    """Groups of `group` (32 or 128) consecutive values along each row.

    X[R][C] -> (q[R][C] uint8, s[R][C/group] E8M0 bytes)."""
    assert group in MX_GROUPS
    x = _as_f32(x)
    R, C = x.shape
    assert C % group == 0
    q, s = _mx_groups_last_axis(x.reshape(R, C // group, group))
    return q.reshape(R, C), s.reshape(R, C // group)


def quantize_mx_act_transposed(x, group=128):
    """Groups of `group` tokens per channel, written transposed.

    X[M][C] -> (qt[C][M] uint8, st[C][M/group] E8M0 bytes); the group of
    channel c and token block b is X[group*b : group*(b+1), c].  Computed on
    the columns directly (not through quantize_mx_act of a transposed copy)."""
    assert group in MX_GROUPS
    x = _as_f32(x)
    M, C = x.shape
    assert M % group == 0
    g = x.reshape(M // group, group, C)  # [b][i][c]
    amax = np.max(np.abs(g), axis=1).astype(np.float32)  # [b][c]
    e = pow2_exponent(amax)
    y = (g.astype(np.float64) * np.exp2(-e.astype(np.float64))[:, None, :]).astype(np.float32)
    q = e4m3_encode(y).reshape(M, C)
    st = (e + E8M0_BIAS).astype(np.uint8).T  # [c][b]
    return np.ascontiguousarray(q.T), np.ascontiguousarray(st)


def quantize_mx_weight(w):
    """128x128 blocks with power-of-two scales; edge blocks may be partial
    (their scale comes from their valid elements only).

    W[N][K] -> (q[N][K] uint8, s[ceil(N/128)][ceil(K/128)] E8M0 bytes)."""
    w = _as_f32(w)
    N, K = w.shape
    nb, kb = -(-N // 128), -(-K // 128)
    q = np.zeros((N, K), dtype=np.uint8)
    s = np.zeros((nb, kb), dtype=np.uint8)
    for i in range(nb):
        for j in range(kb):
            blk = w[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)]
            bq, bs = quantize_mx_group(blk)
            q[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)] = bq
            s[i, j] = bs
    return q, s


_MODE_GROUP = {"act": 128, "mx32": 32}


def logical_mx_operand(q, s, role, trans, mode):
    """Codes and per-element E8M0 scales (as float64 powers of two) of one
    stored operand, in logical orientation (A: [M][K], B: [K][N]).

    role 'A' (logical [M][K]) or 'B' (logical [K][N]); trans 'N' or 'T' as in
    gemm.py; mode 'act' (1x128 along K), 'mx32' (1x32 along K) or 'block'
    (128x128, ceil-divided grid)."""
    q = np.asarray(q, dtype=np.uint8)
    sc = e8m0_decode(s)
    R, C = q.shape
    if role == "A":
        k_axis = 1 if trans == "N" else 0
    else:
        k_axis = 0 if trans == "N" else 1
    if mode in _MODE_GROUP:
        gsz = _MODE_GROUP[mode]
        exp_shape = (R, C // gsz) if k_axis == 1 else (R // gsz, C)
        assert sc.shape == exp_shape, (sc.shape, exp_shape)
        full = np.repeat(sc, gsz, axis=k_axis)
    elif mode == "block":
        assert sc.shape == (-(-R // 128), -(-C // 128)), sc.shape
        full = np.repeat(np.repeat(sc, 128, axis=0), 128, axis=1)[:R, :C]
    else:
        raise ValueError(mode)
    if trans == "T":
        return q.T, full.T
    return q, full


def dequantize_mx_operand(q, s, role, trans, mode):
    """Dequantise one stored operand with E8M0 scales, in logical orientation
    (arguments as for logical_mx_operand): decoded code times its scale."""
    codes, scales = logical_mx_operand(q, s, role, trans, mode)
    return e4m3_decode(codes) * scales


def gemm_mx_ref(layout, qa, sa, mode_a, qb, sb, mode_b):
    """R[M][N] = dequant(A) @ dequant(B) in float64 with E8M0 scales."""
    a = dequantize_mx_operand(qa, sa, "A", layout[0], mode_a)
    b = dequantize_mx_operand(qb, sb, "B", layout[1], mode_b)
    assert a.shape[1] == b.shape[0]
    return np.matmul(a, b)
