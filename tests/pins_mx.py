"""Independent checks ("pins") for the power-of-two (E8M0) oracle in oracle/mx.py.

As in pins.py, each check takes the implementation under test as an argument
so the same check pins the oracle and is shown to reject planted mistakes
(tests/test_oracle_mutants.py).  The checks use exact rational comparisons,
the library E4M3 cast, the fp32-scale oracle on the cases where both rules
must agree, and invariants that follow from the definitions.
"""

from fractions import Fraction

import numpy as np

from pins import library_encode, torch_decode_all


def _frac_pow2(e):
    return Fraction(2) ** int(e)


def amax_samples(rng):
    """float32 amax values: random magnitudes over the whole normal range,
    every 448 * 2**k boundary with its float32 neighbours, and zero."""
    rand = (rng.random(400) + 0.5) * np.exp2(rng.integers(-120, 120, 400))
    edges = []
    for k in range(-126, 120):
        b = np.float32(448.0 * 2.0 ** k)
        if np.isfinite(b) and b > 0:
            edges += [b, np.nextafter(b, np.float32(np.inf)), np.nextafter(b, np.float32(0))]
    vals = np.concatenate([rand.astype(np.float32), np.array(edges, np.float32),
                           np.array([0.0, 1.0, 448.0, 3.4e38, 2.0 ** -126], np.float32)])
    return vals[np.isfinite(vals)]


def check_pow2_exponent(exp_fn, rng):
    """e is the least integer with 448 * 2**e >= amax (exact rationals),
    clamped to [-127, 127]; zero maps to 0."""
    a = amax_samples(rng)
    e = np.asarray(exp_fn(a))
    for v, ev in zip(a.tolist(), e.tolist()):
        assert -127 <= ev <= 127, (v, ev)
        if v == 0:
            assert ev == 0
            continue
        fv = Fraction(v)
        if ev < 127:
            assert fv <= 448 * _frac_pow2(ev), (v, ev)
        if ev > -127:
            assert fv > 448 * _frac_pow2(ev - 1), (v, ev)


def check_mx_scale_invariance(quant_group_fn, rng, group, n=60):
    """Scaling a group by 2**j keeps the codes and adds j to the scale byte."""
    for _ in range(n):
        x = (rng.standard_normal(group) * np.exp(rng.standard_normal())).astype(np.float32)
        q0, b0 = quant_group_fn(x)
        for j in (-30, -3, -1, 1, 4, 30):
            q1, b1 = quant_group_fn((x * np.float32(2.0 ** j)).astype(np.float32))
            assert (q1 == q0).all(), j
            assert int(b1) == int(b0) + j, (j, b0, b1)


def check_mx_fill(quant_group_fn, rng, group, n=200):
    """No element saturates and the largest one lands in (224, 448]: the
    rounded-up power of two leaves at most one binade of headroom."""
    dec = torch_decode_all()
    for _ in range(n):
        x = (rng.standard_t(3, group) * 2.0 ** rng.integers(-40, 40)).astype(np.float32)
        q, b = quant_group_fn(x)
        m = np.max(np.abs(dec[q]))
        assert 224.0 <= m <= 448.0, (m, b)
        # the amax element itself decodes above 224 (or rounds up to 224 exactly)
        i = int(np.argmax(np.abs(x)))
        assert abs(dec[q[i]]) >= 224.0


def check_mx_roundtrip_bound(quant_group_fn, rng, group, n=200):
    """|dec(q) * 2**(b-127) - x| is within half a step of E4M3 at x's
    magnitude: <= (2**-4 + 2**-20)|x| in the normal range, <= 2**-10 * 2**e
    below it.  A scale that is too small (saturation) breaks this."""
    dec = torch_decode_all()
    for _ in range(n):
        x = (rng.standard_t(3, group) * 2.0 ** rng.integers(-30, 30)).astype(np.float32)
        q, b = quant_group_fn(x)
        s = 2.0 ** (int(b) - 127)
        xd = x.astype(np.float64)
        err = np.abs(dec[q] * s - xd)
        normal = np.abs(xd) / s >= 2.0 ** -6
        bound = np.where(normal, (2.0 ** -4 + 2.0 ** -20) * np.abs(xd), 2.0 ** -10 * s)
        assert (err <= bound).all(), np.max(err / bound)


def check_mx_codes_are_library_cast(quant_group_fn, rng, group, n=200):
    """Given the scale byte b, the codes are the library RNE cast of x * 2**(127 - b)."""
    for _ in range(n):
        x = (rng.standard_t(3, group) * 2.0 ** rng.integers(-20, 20)).astype(np.float32)
        q, b = quant_group_fn(x)
        y = (x.astype(np.float64) * 2.0 ** (127 - int(b))).astype(np.float32)
        assert (q == library_encode(y)).all()


def check_mx_exact_representability(quant_group_fn, rng, group, n=100):
    """E4M3 values times 2**j with +-448*2**j present round-trip exactly and
    get the byte 127 + j."""
    finite = torch_decode_all()[:127]
    for _ in range(n):
        j = int(rng.integers(-60, 60))
        v = rng.choice(finite, group) * rng.choice([-1.0, 1.0], group)
        v[int(rng.integers(group))] = 448.0 * rng.choice([-1.0, 1.0])
        x = (v * 2.0 ** j).astype(np.float32)
        q, b = quant_group_fn(x)
        assert int(b) == 127 + j
        assert (torch_decode_all()[q] * 2.0 ** j == x.astype(np.float64)).all()


def check_mx_agrees_with_fp32_rule_on_pow2_amax(quant_group_mx, quant_group_fp32, rng, group, n=100):
    """When amax is 448 * 2**j exactly, amax/448 is already a power of two:
    the fp32-scale rule and the power-of-two rule must give the same codes."""
    for _ in range(n):
        j = int(rng.integers(-30, 30))
        x = (rng.uniform(-1, 1, group) * 448.0 * 2.0 ** j).astype(np.float32)
        x[int(rng.integers(group))] = np.float32(448.0 * 2.0 ** j)
        q1, b = quant_group_mx(x)
        q2, s = quant_group_fp32(x)
        assert np.float32(s) == np.float32(2.0 ** j) and int(b) == 127 + j
        assert (q1 == q2).all()


def check_mx_zero_group(quant_group_fn, group):
    x = np.zeros(group, np.float32)
    x[::3] = -0.0
    q, b = quant_group_fn(x)
    assert int(b) == 127
    assert (q[::3] == 0x80).all() and (q[1::3] == 0x00).all()


def check_mx_group_locality(quant_act_fn, rng, group):
    """Changing one element changes the codes and scale of its own group of
    `group` consecutive row elements only."""
    x = rng.standard_normal((3, 4 * group)).astype(np.float32)
    q0, s0 = quant_act_fn(x, group)
    r, c = 1, int(rng.integers(4 * group))
    x2 = x.copy()
    x2[r, c] = np.float32(1e6)
    q1, s1 = quant_act_fn(x2, group)
    g = c // group
    changed = np.argwhere(q1 != q0)
    assert (changed[:, 0] == r).all() and (changed[:, 1] // group == g).all()
    assert (s1[r, g] != s0[r, g])
    mask = np.ones_like(s0, bool)
    mask[r, g] = False
    assert (s1[mask] == s0[mask]).all()


def fraction_gemm_mx(layout, qa, sa, mode_a, qb, sb, mode_b):
    """Brute-force exact rational sum over every (m, n, k) with E8M0 scales;
    tiny shapes only.  mode: 'act' (1x128 along K), 'mx32' (1x32 along K),
    'block' (128x128)."""
    dec = torch_decode_all()
    A = dec[np.asarray(qa, np.uint8)]
    B = dec[np.asarray(qb, np.uint8)]
    A = A if layout[0] == "N" else A.T
    B = B if layout[1] == "N" else B.T
    M, K = A.shape
    N = B.shape[1]
    gsz = {"act": 128, "mx32": 32}

    def sA(m, k):
        if mode_a == "block":
            return sa[m // 128, k // 128] if layout[0] == "N" else sa[k // 128, m // 128]
        kb = k // gsz[mode_a]
        return sa[m, kb] if layout[0] == "N" else sa[kb, m]

    def sB(k, n):
        if mode_b == "block":
            return sb[k // 128, n // 128] if layout[1] == "N" else sb[n // 128, k // 128]
        kb = k // gsz[mode_b]
        return sb[kb, n] if layout[1] == "N" else sb[n, kb]

    out = np.zeros((M, N), np.float64)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += (Fraction(float(A[m, k])) * _frac_pow2(int(sA(m, k)) - 127)
                        * Fraction(float(B[k, n])) * _frac_pow2(int(sB(k, n)) - 127))
            out[m, n] = float(acc)
    return out


def random_mx_operands(rng, layout, mode_a, mode_b, M, N, K):
    """Random finite codes and E8M0 bytes in the stored layouts."""
    def codes(shape):
        q = rng.integers(0, 256, shape).astype(np.uint8)
        q[(q & 0x7F) == 0x7F] = 0x38
        return q

    def scales(shape, k_axis, mode):
        if mode == "block":
            ss = (-(-shape[0] // 128), -(-shape[1] // 128))
        else:
            ss = list(shape)
            ss[k_axis] //= {"act": 128, "mx32": 32}[mode]
        return rng.integers(120, 135, tuple(ss)).astype(np.uint8)

    a_shape = (M, K) if layout[0] == "N" else (K, M)
    b_shape = (K, N) if layout[1] == "N" else (N, K)
    qa, qb = codes(a_shape), codes(b_shape)
    sa = scales(a_shape, 1 if layout[0] == "N" else 0, mode_a)
    sb = scales(b_shape, 0 if layout[1] == "N" else 1, mode_b)
    return qa, sa, qb, sb


def check_mx_weight_transpose(quant_weight_fn, rng):
    """128x128 blocks commute with transposition: the codes and scales of
    W^T are those of W, transposed (ragged shapes included)."""
    for shape in [(300, 200), (256, 384), (129, 1), (1, 130)]:
        w = (rng.standard_t(3, shape) * 0.02).astype(np.float32)
        q, s = quant_weight_fn(w)
        qt, st = quant_weight_fn(np.ascontiguousarray(w.T))
        assert (q == qt.T).all(), ("codes", shape)
        assert (s == st.T).all(), ("scales", shape)


def check_mx_weight_single_row(quant_weight_fn, quant_act_fn, rng):
    """A block with one non-zero row (not its first) quantises as that row's
    1x128 group; the all-zero blocks get the zero-group scale (byte 127)."""
    w = np.zeros((384, 384), np.float32)
    r = 128 + 1 + int(rng.integers(0, 126))
    row = (rng.standard_normal(128) * rng.uniform(1e-3, 1e3)).astype(np.float32)
    w[r, 256:384] = row
    q, s = quant_weight_fn(w)
    qa, sa = quant_act_fn(row[None, :], 128)
    assert s[1, 2] == sa[0, 0]
    assert (q[r, 256:384] == qa[0]).all()
    blk = q[128:256, 256:384].copy()
    blk[r - 128] = 0
    assert (blk == 0).all()
    others = np.ones(s.shape, bool)
    others[1, 2] = False
    assert (s[others] == 127).all()
