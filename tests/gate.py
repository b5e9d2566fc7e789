"""The GEMM parity gate as the tests apply it (see oracle/tolerance.py).

Every GEMM output C is compared with the oracle's float64 product R of the
dequantised operands under |C - R| <= 1e-2 |R| + (1 + 2**-9) E, E the
bound derived from the matrix core's measured arithmetic.  The survey's O6
figure, max |C - R| / max(|R|, 1e-2 rms(R)), is computed beside it and
printed, not gated.
"""
import numpy as np

import oracle
from oracle import tolerance as tol


def operand_parts(layout, qa, sa, ma, qb, sb, mb, mx=False):
    """Logical (codes, per-element scales) of A [M][K] and B [K][N] from the
    stored operands, for ragged M / N too."""
    logical = oracle.logical_mx_operand if mx else oracle.logical_operand
    qa, sa, qb, sb = (np.asarray(v) for v in (qa, sa, qb, sb))
    # ragged block grids: pad the stored operands so that every block is whole
    a_mn_axis = 0 if layout[0] == "N" else 1
    b_mn_axis = 1 if layout[1] == "N" else 0
    M, N = qa.shape[a_mn_axis], qb.shape[b_mn_axis]

    def padded(q, s, mode, axis):
        ext = q.shape[axis]
        full = -(-ext // 128) * 128
        if full == ext:
            return q, s
        pw = [(0, 0), (0, 0)]
        pw[axis] = (0, full - ext)
        q = np.pad(q, pw)
        if mode not in ("block",):
            s = np.pad(s, pw, constant_values=127 if mx else 1.0)
        return q, s

    qa2, sa2 = padded(qa, sa, ma, a_mn_axis)
    qb2, sb2 = padded(qb, sb, mb, b_mn_axis)
    ac, asc = logical(qa2, sa2, "A", layout[0], ma)
    bc, bsc = logical(qb2, sb2, "B", layout[1], mb)
    return ac[:M], asc[:M], bc[:, :N], bsc[:, :N]


def reference(ac, asc, bc, bsc):
    return (oracle.e4m3_decode(ac) * asc) @ (oracle.e4m3_decode(bc) * bsc)


def check(C, ac, asc, bc, bsc, what, R=None, mx=False):
    """Assert the gate for C against the logical operands (mx: the E8M0
    path, whose matrix core accumulates across K blocks); returns
    (bound ratio, O6 figure)."""
    C = np.asarray(C, dtype=np.float64)
    if R is None:
        R = reference(ac, asc, bc, bsc)
    E = tol.gemm_error_bound(ac, asc, bc, bsc, oracle.e4m3_decode, mfma_accumulates=mx)
    ratio = tol.bound_ratio(C, R, E)
    o6 = oracle.o6_error(C, R)
    print(f"[gate] {what}: bound ratio {ratio:.3f}  O6 {o6:.3e}  "
          f"normwise {oracle.normwise_error(C, R):.3e}", flush=True)
    assert ratio <= 1.0, (what, ratio, o6)
    return ratio, o6


def check_stored(C, layout, qa, sa, ma, qb, sb, mb, what, mx=False):
    return check(C, *operand_parts(layout, qa, sa, ma, qb, sb, mb, mx), what, mx=mx)
