"""Planted mistakes in the oracle must be caught by the pins.

Each mutant below is a plausible bug (wrong rounding, wrong format variant,
wrong scale formula, wrong grouping axis, a dropped transpose or scale).  The
test asserts that at least one pin from tests/pins.py rejects it, which shows
the pins that hold for the real oracle are not vacuous.  Everything runs on
the CPU.
"""
import numpy as np
import pytest

import pins
from oracle import e4m3_decode, e4m3_encode, gemm_ref, quantize_act, quantize_act_transposed

DEC = e4m3_decode(np.arange(256, dtype=np.uint8))


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


# ---- codec mutants -------------------------------------------------------

def enc_round_half_away(y):
    y = np.asarray(y, np.float32)
    out = e4m3_encode(y)
    # replace ties-to-even by ties-away on exact midpoints
    a = np.abs(y.astype(np.float64))
    lo = e4m3_encode(np.nextafter(np.abs(y), np.float32(0)))
    hi = e4m3_encode(np.nextafter(np.abs(y), np.float32(np.inf)))
    mid = (lo != hi) & (np.abs(DEC[lo & 0x7F] - a) == np.abs(DEC[hi & 0x7F] - a))
    return np.where(mid, hi | (out & 0x80), out).astype(np.uint8)


def enc_fnuz_max240(y):
    y = np.clip(np.asarray(y, np.float32), -240.0, 240.0)
    return e4m3_encode(y)


def enc_truncate(y):
    y = np.asarray(y, np.float32)
    out = e4m3_encode(y)
    back = DEC[out & 0x7F]
    over = back > np.abs(y.astype(np.float64))
    return np.where(over & ((out & 0x7F) > 0), out - 1, out).astype(np.uint8)


@pytest.mark.parametrize("mutant", [enc_round_half_away, enc_fnuz_max240, enc_truncate])
def test_codec_mutants_are_caught(mutant):
    assert _fails(pins.check_encode_points, mutant, pins.critical_points())


# ---- quantiser mutants ---------------------------------------------------

def _group(x, denom=448.0, mult_by_scale=False, fmt_max=448.0):
    x = np.asarray(x, np.float32)
    amax = np.float32(np.max(np.abs(x)))
    if amax == 0:
        return e4m3_encode(x), np.float32(1)
    s = np.float32(amax / np.float32(denom))
    inv = s if mult_by_scale else np.float32(np.float32(denom) / amax)
    return e4m3_encode(np.clip(x * inv, -fmt_max, fmt_max)), s


def q_denominator_447(x):
    return _group(x, denom=447.0)


def q_mult_by_scale(x):
    return _group(x, mult_by_scale=True)


def q_scale_for_240(x):
    return _group(x, denom=240.0, fmt_max=240.0)


def q_nonzero_scale_for_zero_group(x):
    x = np.asarray(x, np.float32)
    if np.max(np.abs(x)) == 0:
        return e4m3_encode(x), np.float32(0.0)
    return _group(x)


@pytest.mark.parametrize("mutant", [q_denominator_447, q_mult_by_scale, q_scale_for_240,
                                    q_nonzero_scale_for_zero_group])
def test_quantiser_mutants_are_caught(mutant):
    rng = np.random.default_rng(0)
    caught = (_fails(pins.check_amax_maps_to_448, mutant, rng)
              or _fails(pins.check_exact_representability, mutant, DEC, rng)
              or _fails(pins.check_roundtrip_bound, mutant, rng)
              or _fails(pins.check_zero_group, mutant))
    assert caught


def test_transposed_grouping_mutant_is_caught():
    # groups taken along the channel axis instead of the token axis
    def bad_transposed(x):
        q, s = quantize_act(x)  # groups along channels
        return np.ascontiguousarray(q.T), None

    rng = np.random.default_rng(1)
    x = rng.standard_t(3, (256, 256)).astype(np.float32)
    qt, _ = quantize_act_transposed(x)
    qb, _ = bad_transposed(x)
    q2, _ = quantize_act(np.ascontiguousarray(x.T))
    assert (qt == q2).all() and not (qb == q2).all()


# ---- GEMM mutants --------------------------------------------------------

def gemm_dropped_b_scale(layout, qa, sa, ma, qb, sb, mb):
    return gemm_ref(layout, qa, sa, ma, qb, np.ones_like(sb), mb)


def gemm_transposed_block_grid(layout, qa, sa, ma, qb, sb, mb):
    if mb == "block" and sb.shape[0] == sb.shape[1]:
        sb = np.ascontiguousarray(sb.T)
    return gemm_ref(layout, qa, sa, ma, qb, sb, mb)


@pytest.mark.parametrize("mutant", [gemm_dropped_b_scale, gemm_transposed_block_grid])
def test_gemm_mutants_are_caught(mutant):
    rng = np.random.default_rng(2)
    qa, sa, qb, sb = pins.integer_exact_operands(rng, "NT", "act", "block", 256, 256, 256)
    E = pins.exact_gemm_int("NT", qa, sa, "act", qb, sb, "block")
    assert (gemm_ref("NT", qa, sa, "act", qb, sb, "block") == E).all()
    assert not (mutant("NT", qa, sa, "act", qb, sb, "block") == E).all()


def test_gemm_wrong_operand_orientation_is_caught():
    rng = np.random.default_rng(3)
    qa, sa, qb, sb = pins.integer_exact_operands(rng, "NN", "act", "block", 256, 256, 256)
    E = pins.exact_gemm_int("NN", qa, sa, "act", qb, sb, "block")
    # reading the NN operand as if it were NT (B stored [N][K]) is a transpose bug
    wrong = gemm_ref("NT", qa, sa, "act", qb, np.ascontiguousarray(sb.T), "block")
    assert not (wrong == E).all()


# ---- power-of-two (E8M0) mutants -------------------------------------------

import pins_mx  # noqa: E402
from oracle import pow2_exponent, quantize_group, quantize_mx_act  # noqa: E402


def exp_floor(a):
    """floor(log2(amax/448)) instead of rounding up: the OCP MX default."""
    a = np.asarray(a, np.float64)
    e = np.where(a == 0, 0, np.floor(np.log2(np.where(a == 0, 1, a) / 448.0)))
    return np.clip(e, -127, 127).astype(np.int64)


def exp_no_clamp_high(a):
    """Rounds to the nearest power instead of up (log2 rounded half-up)."""
    a = np.asarray(a, np.float64)
    e = np.where(a == 0, 0, np.round(np.log2(np.where(a == 0, 1, a) / 448.0)))
    return np.clip(e, -127, 127).astype(np.int64)


@pytest.mark.parametrize("mutant", [exp_floor, exp_no_clamp_high])
def test_pow2_exponent_mutants_are_caught(mutant):
    assert _fails(pins_mx.check_pow2_exponent, mutant, np.random.default_rng(0))


def _mx_group(x, exp_fn=pow2_exponent, bias=127, saturate_ok=True):
    x = np.asarray(x, np.float32)
    amax = np.float32(np.max(np.abs(x)))
    e = int(exp_fn(np.array([amax], np.float32))[0])
    y = (x.astype(np.float64) * 2.0 ** -e).astype(np.float32)
    return e4m3_encode(y), np.uint8(e + bias)


def mxq_floor_exponent(x):
    return _mx_group(x, exp_fn=exp_floor)


def mxq_bias_128(x):
    return _mx_group(x, bias=128)


def mxq_fp32_rule(x):
    """Uses the fp32 amax/448 scale but reports its rounded-up exponent."""
    q, s = quantize_group(x)
    e = int(pow2_exponent(np.array([np.max(np.abs(np.asarray(x, np.float32)))], np.float32))[0])
    return q, np.uint8(e + 127)


@pytest.mark.parametrize("mutant", [mxq_floor_exponent, mxq_bias_128, mxq_fp32_rule])
def test_mx_quantiser_mutants_are_caught(mutant):
    r = np.random.default_rng(1)
    caught = (_fails(pins_mx.check_mx_fill, mutant, r, 32)
              or _fails(pins_mx.check_mx_exact_representability, mutant, r, 32)
              or _fails(pins_mx.check_mx_codes_are_library_cast, mutant, r, 32)
              or _fails(pins_mx.check_mx_roundtrip_bound, mutant, r, 32))
    assert caught


def mx_act_groups_misaligned(x, group):
    """Groups of `group` starting at column 16 (a wrong group origin)."""
    x = np.asarray(x, np.float32)
    rolled = np.roll(x, -16, axis=1)
    q, s = quantize_mx_act(rolled, group)
    return np.roll(q, 16, axis=1), s


def test_mx_group_origin_mutant_is_caught():
    assert _fails(pins_mx.check_mx_group_locality, mx_act_groups_misaligned,
                  np.random.default_rng(2), 32)


def gemm_mx32_scales_on_wrong_axis(layout, qa, sa, ma, qb, sb, mb):
    """A's 1x32 scales applied to permuted K positions (a group/position mix-up)."""
    from oracle import dequantize_mx_operand, e8m0_decode
    full = np.repeat(e8m0_decode(sa), 32, axis=1)
    perm = np.random.default_rng(9).permutation(full.shape[1])
    a = e4m3_decode(qa) * full[:, perm]
    return a @ dequantize_mx_operand(qb, sb, "B", layout[1], mb)


def test_mx_gemm_scale_axis_mutant_is_caught():
    M, N, K = 4, 3, 128
    qa, sa, qb, sb = pins_mx.random_mx_operands(np.random.default_rng(3), "NT", "mx32", "mx32",
                                                M, N, K)
    want = pins_mx.fraction_gemm_mx("NT", qa, sa, "mx32", qb, sb, "mx32")
    got = gemm_mx32_scales_on_wrong_axis("NT", qa, sa, "mx32", qb, sb, "mx32")
    assert not np.allclose(got, want, rtol=0, atol=1e-12 * np.max(np.abs(want)))


# ---- E8M0 weight-quantiser mutants ------------------------------------------

from oracle import quantize_mx_group, quantize_mx_weight  # noqa: E402


def mxw_first_row_amax(w):
    """Each block's scale taken from its first row's amax only."""
    w = np.asarray(w, np.float32)
    q, s = quantize_mx_weight(w)
    for i in range(s.shape[0]):
        for j in range(s.shape[1]):
            blk = w[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)]
            e = pow2_exponent(np.max(np.abs(blk[0])))
            y = (blk.astype(np.float64) * np.exp2(-float(e))).astype(np.float32)
            q[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)] = e4m3_encode(np.clip(y, -448, 448))
            s[i, j] = np.uint8(e + 127)
    return q, s


def mxw_row_strips(w):
    """1x128 groups along each row instead of 128x128 blocks, the scale of
    the block taken from the block's first row group."""
    w = np.asarray(w, np.float32)
    N, K = w.shape
    q = np.zeros((N, K), np.uint8)
    s = np.zeros((-(-N // 128), -(-K // 128)), np.uint8)
    for r in range(N):
        for j in range(-(-K // 128)):
            qg, bg = quantize_mx_group(w[r, 128 * j:128 * (j + 1)])
            q[r, 128 * j:128 * (j + 1)] = qg
            if r % 128 == 0:
                s[r // 128, j] = bg
    return q, s


@pytest.mark.parametrize("mutant", [mxw_first_row_amax, mxw_row_strips])
def test_mx_weight_mutants_are_caught(mutant):
    r = np.random.default_rng(3)
    caught = (_fails(pins_mx.check_mx_weight_transpose, mutant, r)
              or _fails(pins_mx.check_mx_weight_single_row, mutant, quantize_mx_act, r))
    assert caught
