"""Float64 reference of the blockwise-FP8 GEMM.

What the GPU computes, per the Puro-2B paper translation
(papers.lianghsun.dev), section 3.2, with the DeepSeek-V3 fine-grained
design it follows: C[m][n] = sum over K blocks kb of
(sum_{k in kb} dec(A)[m][k] * dec(B)[k][n]) * sA * sB, where sA and sB are
the scales of the groups/blocks the elements belong to; fp32 partials are
promoted once per 128-deep block and the result is stored as bfloat16.

The reference below is the plain definition: dequantise both operands to
float64 (value = code * scale, the MXFP figure's decode rule in the Puro-2B
tutorial, bloombook.cn) and multiply with numpy.matmul in float64.  Every
dequantised value is exact in float64 (at most 4 + 24 significant bits).

Layout letters describe row-major storage (a reading; the pages do not
name an API):
  A 'N' stored [M][K];  A 'T' stored [K][M]
  B 'N' stored [K][N];  B 'T' stored [N][K]
Scale tensors follow the stored orientation:
  act mode (1x128 along K): the stored K axis is divided by 128
  block mode (128x128):     both stored axes are divided by 128
"""

import numpy as np

from .e4m3 import e4m3_decode

GROUP = 128


def logical_operand(q, s, role, trans, mode):
    """Codes and per-element scales of one stored operand, in logical
    orientation (A: [M][K], B: [K][N]).

    role: 'A' (logical [M][K]) or 'B' (logical [K][N]).
    trans: 'N' or 'T' (see module docstring).
    mode: 'act' (1x128 groups along K) or 'block' (128x128).
    Returns (codes uint8, scales float64), both in logical orientation; the
    dequantised operand is their elementwise product (value = code * scale).
    """
    q = np.asarray(q, dtype=np.uint8)
    s = np.asarray(s, dtype=np.float32).astype(np.float64)
    R, C = q.shape
    if role == "A":
        k_axis = 1 if trans == "N" else 0
    else:
        k_axis = 0 if trans == "N" else 1
    if mode == "act":
        exp_shape = (R, C // GROUP) if k_axis == 1 else (R // GROUP, C)
        assert s.shape == exp_shape, (s.shape, exp_shape)
        full = np.repeat(s, GROUP, axis=k_axis)
    elif mode == "block":
        assert s.shape == (R // GROUP, C // GROUP), s.shape
        full = np.repeat(np.repeat(s, GROUP, axis=0), GROUP, axis=1)
    else:
        raise ValueError(mode)
    if trans == "T":
        return q.T, full.T
    return q, full


def dequantize_operand(q, s, role, trans, mode):
    """Dequantise one stored operand and return it in logical orientation
    (arguments as for logical_operand): decoded code times its scale."""
    codes, scales = logical_operand(q, s, role, trans, mode)
    return e4m3_decode(codes) * scales


def gemm_ref(layout, qa, sa, mode_a, qb, sb, mode_b):
    """R[M][N] = dequant(A) @ dequant(B) in float64.  layout e.g. 'NT'."""
    ta, tb = layout[0], layout[1]
    a = dequantize_operand(qa, sa, "A", ta, mode_a)
    b = dequantize_operand(qb, sb, "B", tb, mode_b)
    assert a.shape[1] == b.shape[0]
    return np.matmul(a, b)


def o6_error(c, r):
    """The elementwise relative error with a 1e-2 * rms(R) floor:
    max |C - R| / max(|R|, 1e-2 * rms(R)).

    Reported beside the parity gate (oracle.tolerance), not a gate itself:
    an output whose exact value cancels far below the size of its terms has
    an absolute error set by those terms (the matrix core's alignment of
    each group of products), so this ratio is unbounded for such outputs.
    """
    c = np.asarray(c, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if r.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    den = np.maximum(np.abs(r), 1e-2 * rms)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(c - r) / den))


def normwise_error(c, r):
    """max|C-R| / max|R| (reported beside the gate, not a gate)."""
    c = np.asarray(c, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    m = float(np.max(np.abs(r))) if r.size else 0.0
    return float(np.max(np.abs(c - r))) / m if m > 0 else float(np.max(np.abs(c - r), initial=0.0))
