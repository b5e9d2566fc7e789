"""Pins for the oracle's quantisers (CPU only).

Closed-form invariants that the definitions fix (amax maps to +-448, scale
invariance under powers of two, exact representability of E4M3 data, the
round-trip error bound, the all-zero group) and cross-identities between the
three quantisers, each computed by separate code in the oracle.
"""
import numpy as np
import torch

import pins
from oracle import (e4m3_decode, quantize_act, quantize_act_transposed,
                    quantize_group, quantize_weight)
from workloads import bf16_bits


def rng(seed=0):
    return np.random.default_rng(seed)


def test_amax_maps_to_448():
    pins.check_amax_maps_to_448(quantize_group, rng(1))


def test_scale_invariance():
    pins.check_scale_invariance(quantize_group, rng(2))


def test_exact_representability():
    pins.check_exact_representability(quantize_group, e4m3_decode(np.arange(256, dtype=np.uint8)), rng(3))


def test_roundtrip_bound():
    pins.check_roundtrip_bound(quantize_group, rng(4))


def test_zero_group():
    pins.check_zero_group(quantize_group)


def test_scale_is_ieee_division():
    # s must be the float32 quotient amax/448 computed by the library
    r = rng(5)
    for _ in range(200):
        x = (r.standard_normal(128) * 10.0 ** r.uniform(-8, 8)).astype(np.float32)
        _, s = quantize_group(x)
        amax = torch.from_numpy(np.abs(x)).max()
        assert np.float32(s) == (amax / torch.tensor(448.0, dtype=torch.float32)).item()


def test_act_groups_are_rows_of_128():
    r = rng(6)
    x = r.standard_normal((8, 512)).astype(np.float32)
    q, s = quantize_act(x)
    assert q.shape == (8, 512) and s.shape == (8, 4)
    for i in range(8):
        for g in range(4):
            qg, sg = quantize_group(x[i, 128 * g:128 * g + 128])
            assert (q[i, 128 * g:128 * g + 128] == qg).all() and s[i, g] == sg


def test_transposed_equals_act_on_transpose():
    r = rng(7)
    x = (r.standard_t(3, (384, 256)) * 3).astype(np.float32)
    x[:, 5] = 0.0  # an all-zero token-axis group
    qt, st = quantize_act_transposed(x)
    q2, s2 = quantize_act(np.ascontiguousarray(x.T))
    assert qt.shape == (256, 384) and st.shape == (256, 3)
    assert (qt == q2).all()
    assert (st.view(np.uint32) == s2.view(np.uint32)).all()


def test_weight_transpose_identity():
    r = rng(8)
    w = (r.standard_normal((256, 384)) * 0.02).astype(np.float32)
    q, s = quantize_weight(w)
    qT, sT = quantize_weight(np.ascontiguousarray(w.T))
    assert (q == qT.T).all()
    assert (s.view(np.uint32) == sT.T.view(np.uint32)).all()


def test_weight_single_row_block_equals_act():
    r = rng(9)
    w = np.zeros((128, 256), np.float32)
    w[37] = r.standard_normal(256).astype(np.float32)
    q, s = quantize_weight(w)
    qa, sa = quantize_act(w[37:38])
    assert (q[37] == qa[0]).all()
    assert s[0, 0] == sa[0, 0] and s[0, 1] == sa[0, 1]
    assert (np.delete(q, 37, axis=0) == 0).all()


def test_weight_blocks_are_128x128():
    r = rng(10)
    w = r.standard_normal((256, 256)).astype(np.float32)
    q, s = quantize_weight(w)
    for bi in range(2):
        for bj in range(2):
            blk = w[128 * bi:128 * bi + 128, 128 * bj:128 * bj + 128]
            qb, sb = quantize_group(blk)
            assert (q[128 * bi:128 * bi + 128, 128 * bj:128 * bj + 128] == qb).all()
            assert s[bi, bj] == sb


def test_bf16_input_equals_fp32_input():
    g = torch.Generator().manual_seed(11)
    xb = torch.randn(64, 256, generator=g).to(torch.bfloat16)
    q1, s1 = quantize_act(bf16_bits(xb))
    q2, s2 = quantize_act(xb.float().numpy())
    assert (q1 == q2).all() and (s1 == s2).all()
    qt1, st1 = quantize_act_transposed(bf16_bits(xb.T.contiguous()))
    qt2, st2 = quantize_act_transposed(xb.T.contiguous().float().numpy())
    assert (qt1 == qt2).all() and (st1 == st2).all()


def test_divide_reading_differs_rarely():
    # The alternative element map fl32(x / s) differs from fl32(x * inv) only
    # in rare last-bit cases; both satisfy the invariants above.
    r = rng(12)
    x = r.standard_normal((4096, 128)).astype(np.float32)
    diffs = 0
    for row in x:
        a, _ = quantize_group(row)
        b, _ = quantize_group(row, use_divide=True)
        diffs += int((a != b).sum())
    assert diffs < 0.01 * x.size
