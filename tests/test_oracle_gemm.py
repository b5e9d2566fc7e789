"""Pins for the oracle's float64 GEMM reference (CPU only).

(i) integer-exact construction checked against an exact integer sum done
block by block with the library decode; (ii) a one-hot selector; (iii) with
unit scales the reference is numpy.matmul of library-decoded operands;
(iv) brute-force exact rational sums at tiny shapes, for every layout and
scale mode.
"""
import itertools

import numpy as np
import pytest

import pins
from oracle import gemm_ref, quantize_act, quantize_weight

LAYOUTS = ["NT", "NN", "TN"]
MODES = [("act", "block"), ("act", "act"), ("block", "act"), ("block", "block")]


@pytest.mark.parametrize("layout,modes", list(itertools.product(LAYOUTS, MODES)))
def test_integer_exact(layout, modes):
    r = np.random.default_rng(hash((layout, modes)) % 2 ** 32)
    M, N, K = 256, 384, 512
    qa, sa, qb, sb = pins.integer_exact_operands(r, layout, modes[0], modes[1], M, N, K)
    R = gemm_ref(layout, qa, sa, modes[0], qb, sb, modes[1])
    E = pins.exact_gemm_int(layout, qa, sa, modes[0], qb, sb, modes[1])
    assert (R == E).all()


@pytest.mark.parametrize("layout", LAYOUTS)
def test_selector(layout):
    r = np.random.default_rng(3)
    M, N, K = 128, 256, 384
    sel = r.integers(0, K, M)
    A = np.zeros((M, K), np.uint8)
    A[np.arange(M), sel] = 0x38  # 1.0
    sa = r.uniform(0.5, 2, (M, K // 128)).astype(np.float32)
    Bl = r.integers(0, 256, (K, N)).astype(np.uint8)
    Bl[(Bl & 0x7F) == 0x7F] = 0x01  # no NaN codes
    sb = r.uniform(0.5, 2, (K // 128, N // 128)).astype(np.float32)
    qa = A if layout[0] == "N" else np.ascontiguousarray(A.T)
    sa_s = sa if layout[0] == "N" else np.ascontiguousarray(sa.T)
    qb = Bl if layout[1] == "N" else np.ascontiguousarray(Bl.T)
    sb_s = sb if layout[1] == "N" else np.ascontiguousarray(sb.T)
    R = gemm_ref(layout, qa, sa_s, "act", qb, sb_s, "block")
    dec = pins.torch_decode_all()
    for m in range(M):
        k = sel[m]
        exp = dec[Bl[k]] * np.float64(sa[m, k // 128]) * np.repeat(sb[k // 128], 128).astype(np.float64)
        assert (R[m] == exp).all()


def test_unit_scales_is_library_matmul():
    r = np.random.default_rng(4)
    M, N, K = 256, 256, 384
    qa = r.integers(0, 256, (M, K)).astype(np.uint8)
    qb = r.integers(0, 256, (N, K)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0
    qb[(qb & 0x7F) == 0x7F] = 0
    R = gemm_ref("NT", qa, np.ones((M, K // 128), np.float32), "act",
                 qb, np.ones((N // 128, K // 128), np.float32), "block")
    dec = pins.torch_decode_all()
    assert np.allclose(R, dec[qa] @ dec[qb].T, rtol=1e-13, atol=0)


@pytest.mark.parametrize("layout,modes", list(itertools.product(LAYOUTS, MODES)))
def test_bruteforce_fraction(layout, modes):
    r = np.random.default_rng(5)
    # block mode needs the row/column extent to be a multiple of 128 too
    M = 128 if modes[0] == "block" else 3
    N = 128 if modes[1] == "block" else 2
    K = 256
    qa, sa, qb, sb = pins.integer_exact_operands(r, layout, modes[0], modes[1], M, N, K)
    # arbitrary (non power of two) fp32 scales and arbitrary finite codes
    sa = r.uniform(1e-3, 10, sa.shape).astype(np.float32)
    sb = r.uniform(1e-3, 10, sb.shape).astype(np.float32)
    qa = r.integers(0, 256, qa.shape).astype(np.uint8)
    qb = r.integers(0, 256, qb.shape).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x7E
    qb[(qb & 0x7F) == 0x7F] = 0x7E
    R = gemm_ref(layout, qa, sa, modes[0], qb, sb, modes[1])
    if M == 128 and N == 128:
        rows, cols = np.arange(0, 128, 41), np.arange(0, 128, 53)
    else:
        rows, cols = np.arange(M), np.arange(N)
    # brute force on a sub-grid of outputs (rows/cols selected before the sum)
    E = pins.fraction_gemm(layout, qa, sa, modes[0], qb, sb, modes[1]) if M * N <= 6 else None
    if E is not None:
        assert np.max(np.abs(R - E)) <= 1e-12 * np.max(np.abs(E))
    else:
        full = pins.fraction_gemm_points(layout, qa, sa, modes[0], qb, sb, modes[1], rows, cols)
        assert np.max(np.abs(R[np.ix_(rows, cols)] - full)) <= 1e-12 * np.max(np.abs(full))


def test_realistic_quantised_product_close_to_unquantised():
    # The blockwise FP8 product tracks the unquantised fp64 product: a sanity
    # check of the whole oracle chain (not a parity bar).
    r = np.random.default_rng(6)
    x = r.standard_normal((256, 512)).astype(np.float32)
    w = (r.standard_normal((384, 512)) * 0.02).astype(np.float32)
    qa, sa = quantize_act(x)
    qb, sb = quantize_weight(w)
    R = gemm_ref("NT", qa, sa, "act", qb, sb, "block")
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.linalg.norm(R - exact) / np.linalg.norm(exact) < 0.06
