"""Blockwise E4M3 quantisers: 1x128 activation groups and 128x128 weight blocks.

Follows the Puro-2B paper translation (papers.lianghsun.dev), section 3.2
"FP8 mixed-precision training": scales are computed online for each local
group; activations and activation gradients use 1-D groups of 128
consecutive values along the reduction dimension of the GEMM they feed;
weights use 128x128 2-D blocks, each with its own scale.  The decode rule
value = code * scale is the MXFP figure of the Puro-2B tutorial
(bloombook.cn), FP8/MuonH section.

Readings (the pages leave these open):
  * scale s = fl32(amax / 448), an IEEE float32 division;
  * element map y = fl32(x * fl32(448 / amax)), one float32 multiply, then
    saturating round-to-nearest-even to E4M3;
  * amax == 0 gives s = 1.0 and signed zero codes;
  * groups with 0 < amax < 448 * 2**-126 (scale would be subnormal) and
    non-finite inputs are outside the contract.
"""

import numpy as np

from .e4m3 import e4m3_encode

GROUP = 128
_F448 = np.float32(448.0)


def quantize_group(x, use_divide=False):
    """Quantise one group (any shape) of float32 values with a shared scale.

    Returns (codes uint8 with x's shape, scale as numpy float32).

    Steps: amax = max |x| (exact in float32); if amax == 0 the scale is 1.0;
    else s = fl32(amax/448), inv = fl32(448/amax); y = fl32(x*inv) (or
    fl32(x/s) when ``use_divide`` -- an alternative reading kept only for a
    diagnostic test); codes = E4M3 saturating RNE of y.
    """
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    if amax == 0:
        s = np.float32(1.0)
        inv = np.float32(1.0)
    else:
        s = np.float32(amax / _F448)
        inv = np.float32(_F448 / amax)
    if use_divide:
        y = (x / s).astype(np.float32)
    else:
        y = (x * inv).astype(np.float32)
    return e4m3_encode(y), s


def _as_f32(x):
    x = np.asarray(x)
    if x.dtype == np.float32:
        return x
    if x.dtype == np.uint16:  # raw bfloat16 bit patterns
        return (x.astype(np.uint32) << 16).view(np.float32)
    return x.astype(np.float32)


def _quantize_groups_last_axis(g):
    """Group-wise quantisation where each group is g[..., :] (last axis).

    This is quantize_group applied independently to every group; it is
    written vectorised over the groups only because the per-group Python
    loop is too slow at the configuration shapes.  The per-element
    arithmetic is identical (float32 max, divide, multiply; E4M3 RNE).
    """
    amax = np.max(np.abs(g), axis=-1).astype(np.float32)
    zero = amax == 0
    safe = np.where(zero, np.float32(1.0), amax).astype(np.float32)
    s = np.where(zero, np.float32(1.0), (safe / _F448).astype(np.float32))
    inv = np.where(zero, np.float32(1.0), (_F448 / safe).astype(np.float32))
    y = (g * inv[..., None].astype(np.float32)).astype(np.float32)
    return e4m3_encode(y), s.astype(np.float32)


def quantize_act(x):
    """1x128 groups along each row: X[R][C] -> (q[R][C] uint8, s[R][C/128] f32).

    Input: float32, or uint16 holding bfloat16 bit patterns (widened
    exactly).  Group g of row r is X[r, 128g:128g+128].
    """
    x = _as_f32(x)
    R, C = x.shape
    assert C % GROUP == 0
    g = x.reshape(R, C // GROUP, GROUP)
    q, s = _quantize_groups_last_axis(g)
    return q.reshape(R, C), s.reshape(R, C // GROUP)


def quantize_act_transposed(x):
    """Token-axis 1x128 groups for wgrad, written transposed.

    X[M][C] -> (qt[C][M] uint8, st[C][M/128] f32); the group for channel c
    and token block b is X[128b:128b+128, c].  Written directly on columns
    (not by calling quantize_act on a transposed copy) so the identity with
    quantize_act(X.T) is a real check.
    """
    x = _as_f32(x)
    M, C = x.shape
    assert M % GROUP == 0
    g = x.reshape(M // GROUP, GROUP, C)  # [b][i][c]
    amax = np.max(np.abs(g), axis=1).astype(np.float32)  # [b][c]
    zero = amax == 0
    safe = np.where(zero, np.float32(1.0), amax).astype(np.float32)
    s = np.where(zero, np.float32(1.0), (safe / _F448).astype(np.float32))
    inv = np.where(zero, np.float32(1.0), (_F448 / safe).astype(np.float32))
    y = (g * inv[:, None, :].astype(np.float32)).astype(np.float32)
    q = e4m3_encode(y).reshape(M, C)  # natural [m][c] order
    qt = np.ascontiguousarray(q.T)
    st = np.ascontiguousarray(s.T.astype(np.float32))  # [c][b]
    return qt, st


def quantize_weight(w):
    """128x128 blocks: W[N][K] -> (q[N][K] uint8, s[N/128][K/128] f32)."""
    w = _as_f32(w)
    N, K = w.shape
    assert N % GROUP == 0 and K % GROUP == 0
    nb, kb = N // GROUP, K // GROUP
    g = w.reshape(nb, GROUP, kb, GROUP).transpose(0, 2, 1, 3)  # [nb][kb][i][j]
    g = g.reshape(nb, kb, GROUP * GROUP)
    q, s = _quantize_groups_last_axis(g)
    q = q.reshape(nb, kb, GROUP, GROUP).transpose(0, 2, 1, 3).reshape(N, K)
    return np.ascontiguousarray(q), s.reshape(nb, kb)
