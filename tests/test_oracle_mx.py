"""Pins of the power-of-two (E8M0) oracle (CPU only)."""

import numpy as np
import pytest

import oracle
from pins import GROUP
from pins_mx import (
    check_mx_agrees_with_fp32_rule_on_pow2_amax,
    check_mx_codes_are_library_cast,
    check_mx_roundtrip_bound,
    check_mx_exact_representability,
    check_mx_fill,
    check_mx_group_locality,
    check_mx_scale_invariance,
    check_mx_weight_single_row,
    check_mx_weight_transpose,
    check_mx_zero_group,
    check_pow2_exponent,
    fraction_gemm_mx,
    random_mx_operands,
)


def rng(seed=0):
    return np.random.default_rng(seed)


def test_pow2_exponent_is_least_covering_power():
    check_pow2_exponent(oracle.pow2_exponent, rng(1))


def test_e8m0_decode():
    b = np.arange(255, dtype=np.uint8)
    v = oracle.e8m0_decode(b)
    assert v[127] == 1.0 and v[128] == 2.0 and v[126] == 0.5
    assert (v[1:] / v[:-1] == 2.0).all()


@pytest.mark.parametrize("group", [32, 128])
def test_mx_group_invariants(group):
    fn = oracle.quantize_mx_group
    check_mx_scale_invariance(fn, rng(2), group)
    check_mx_fill(fn, rng(3), group)
    check_mx_codes_are_library_cast(fn, rng(4), group)
    check_mx_roundtrip_bound(fn, rng(15), group)
    check_mx_exact_representability(fn, rng(5), group)
    check_mx_zero_group(fn, group)


@pytest.mark.parametrize("group", [32, 128])
def test_mx_agrees_with_fp32_rule_when_amax_is_448_times_pow2(group):
    check_mx_agrees_with_fp32_rule_on_pow2_amax(oracle.quantize_mx_group, oracle.quantize_group,
                                                 rng(6), group)


@pytest.mark.parametrize("group", [32, 128])
def test_mx_act_groups_are_row_runs(group):
    check_mx_group_locality(oracle.quantize_mx_act, rng(7), group)
    x = rng(8).standard_normal((5, 4 * group)).astype(np.float32)
    q, s = oracle.quantize_mx_act(x, group)
    for r in range(5):
        for g in range(4):
            qg, bg = oracle.quantize_mx_group(x[r, g * group:(g + 1) * group])
            assert (q[r, g * group:(g + 1) * group] == qg).all() and s[r, g] == bg


@pytest.mark.parametrize("group", [32, 128])
def test_mx_transposed_equals_act_on_transpose(group):
    x = (rng(9).standard_t(3, (2 * group, 3 * group)) * 0.1).astype(np.float32)
    qt, st = oracle.quantize_mx_act_transposed(x, group)
    q2, s2 = oracle.quantize_mx_act(np.ascontiguousarray(x.T), group)
    assert (qt == q2).all() and (st == s2).all()


def test_mx_weight_blocks_and_ragged_edges():
    w = (rng(10).standard_normal((300, 200)) * 0.02).astype(np.float32)
    q, s = oracle.quantize_mx_weight(w)
    assert s.shape == (3, 2)
    for i in range(3):
        for j in range(2):
            blk = w[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)]
            qb, bb = oracle.quantize_mx_group(blk)
            assert s[i, j] == bb
            assert (q[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)] == qb).all()
    # a full block equals the 1x128 act rule applied to the flattened block
    blk = w[:128, :128]
    q2, b2 = oracle.quantize_mx_group(blk.reshape(-1))
    assert b2 == s[0, 0] and (q2.reshape(128, 128) == q[:128, :128]).all()


def test_mx_weight_transpose_identity():
    check_mx_weight_transpose(oracle.quantize_mx_weight, rng(16))


def test_mx_weight_single_row_block_is_an_act_group():
    for seed in (17, 18, 19):
        check_mx_weight_single_row(oracle.quantize_mx_weight, oracle.quantize_mx_act, rng(seed))


def test_mx_bf16_input_equals_fp32_input():
    import torch
    x = torch.randn(64, 256, generator=torch.Generator().manual_seed(11)).to(torch.bfloat16)
    bits = x.view(torch.uint16).numpy() if hasattr(torch, "uint16") else x.view(torch.int16).numpy().view(np.uint16)
    q1, s1 = oracle.quantize_mx_act(bits, 32)
    q2, s2 = oracle.quantize_mx_act(x.float().numpy(), 32)
    assert (q1 == q2).all() and (s1 == s2).all()


@pytest.mark.parametrize("layout,modes", [
    ("NT", ("act", "block")), ("NT", ("act", "act")), ("NT", ("mx32", "mx32")),
    ("NN", ("act", "block")), ("TN", ("act", "act")), ("NT", ("block", "mx32")),
])
def test_mx_gemm_bruteforce_fraction(layout, modes):
    M, N, K = 5, 3, 256
    qa, sa, qb, sb = random_mx_operands(rng(12), layout, modes[0], modes[1], M, N, K)
    got = oracle.gemm_mx_ref(layout, qa, sa, modes[0], qb, sb, modes[1])
    want = fraction_gemm_mx(layout, qa, sa, modes[0], qb, sb, modes[1])
    assert np.allclose(got, want, rtol=0, atol=1e-12 * np.max(np.abs(want)))


def test_mx_gemm_matches_fp32_scale_reference_on_pow2_scales():
    """With scales that are powers of two, the E8M0 reference equals the
    fp32-scale reference (decoded scales passed as float32)."""
    r = rng(13)
    M, N, K = 64, 48, 512
    qa, sa, qb, sb = random_mx_operands(r, "NT", "act", "act", M, N, K)
    got = oracle.gemm_mx_ref("NT", qa, sa, "act", qb, sb, "act")
    want = oracle.gemm_ref("NT", qa, oracle.e8m0_decode(sa).astype(np.float32), "act",
                           qb, oracle.e8m0_decode(sb).astype(np.float32), "act")
    assert np.array_equal(got, want)


def test_mx32_quantised_product_close_to_unquantised():
    """Quantise-then-multiply with 1x32 groups tracks the float64 product of
    the unquantised inputs (MXFP8 granularity is at least as fine as 1x128)."""
    r = rng(14)
    x = r.standard_normal((64, 512)).astype(np.float32)
    w = (r.standard_normal((96, 512)) * 0.02).astype(np.float32)
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    errs = {}
    for g in (32, 128):
        qx, sx = oracle.quantize_mx_act(x, g)
        qw, sw = oracle.quantize_mx_act(w, g)
        mode = "mx32" if g == 32 else "act"
        got = oracle.gemm_mx_ref("NT", qx, sx, mode, qw, sw, mode)
        errs[g] = oracle.normwise_error(got, exact)
    assert errs[32] < 0.06 and errs[128] < 0.06


def test_pow2_dequantised_value_does_not_depend_on_the_group_in_normal_range():
    """With a power-of-two scale 2**e the quantised value x / 2**e has x's
    own significand, so while it stays in E4M3's normal range its code
    decodes to x rounded to 4 significant bits whatever e is: groups of 32
    and of 128 give the same dequantised element except where one of the two
    scaled values is below the smallest normal, 2**-6.  This is why 1x32 and
    1x128 power-of-two scales quantise realistic data almost identically."""
    r = rng(15)
    x = r.standard_t(3, (256, 1024)).astype(np.float32)
    dec = {}
    sub = {}
    for g in (32, 128):
        q, s = oracle.quantize_mx_act(x, g)
        scale = np.repeat(oracle.e8m0_decode(s), g, axis=1)
        dec[g] = oracle.e4m3_decode(q).astype(np.float64) * scale
        sub[g] = np.abs(x.astype(np.float64)) / scale < 2.0 ** -6
    normal = ~(sub[32] | sub[128])
    assert np.array_equal(dec[32][normal], dec[128][normal])
    # the significand rounding itself: |x - dec| <= 2**-4 |x| in the normal range
    xn = x.astype(np.float64)[normal]
    assert np.all(np.abs(dec[128][normal] - xn) <= 2.0 ** -4 * np.abs(xn))
    # and the elements that differ are few and tiny against their group
    assert (~normal).mean() < 0.01
