"""Independent checks ("pins") for the CPU oracle.

Each check takes the implementation under test as an argument, so the same
check pins the real oracle (tests/test_oracle_*.py) and is shown to fail on
planted mistakes (tests/test_oracle_mutants.py).  Nothing here re-types the
oracle's formulas: the checks use a library cast (torch.float8_e4m3fn), a
brute-force nearest-value search, exact integer/rational arithmetic, or
invariants that follow from the definitions.
"""

from fractions import Fraction

import numpy as np
import torch

GROUP = 128


# ---------------------------------------------------------------- E4M3 codec

def torch_decode_all():
    """Library decode of all 256 codes (float64, NaN where the code is NaN)."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def library_encode(y):
    """Library special case of saturating RNE: clamp to +-448, then torch's cast."""
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32))
    return t.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def bruteforce_encode(y):
    """Nearest finite E4M3 value by exhaustive search; ties go to the even code.

    Candidates are the 127 non-negative finite codes 0x00..0x7E decoded by
    the library; saturation follows because nothing above 448 is a candidate.
    Distances are compared exactly, as integers in units of 2**-149 (every
    float32 and every E4M3 value is an integer multiple of that unit).
    """
    from fractions import Fraction as F

    unit = 2 ** 149
    cands = [int(F(float(v)) * unit) for v in torch_decode_all()[:127]]
    y = np.asarray(y, dtype=np.float32).ravel()
    out = np.empty(y.shape, np.uint8)
    for i, v in enumerate(y.tolist()):
        a = abs(int(F(v) * unit))
        best, pick = None, None
        for code, c in enumerate(cands):
            d = abs(a - c)
            if best is None or d < best or (d == best and code % 2 == 0 and pick % 2 == 1):
                best, pick = d, code
        out[i] = pick | (0x80 if np.signbit(np.float32(v)) else 0)
    return out


def critical_points():
    """Every rounding decision point of E4M3 with its float32 neighbours.

    The code values themselves, the midpoints between adjacent codes, the
    saturation region around 448..480 and the underflow region, each with
    nextafter up/down, plus zeros.  A monotone encoder that is right on all
    of these is right everywhere in between.
    """
    vals = torch_decode_all()[:127]
    mids = (vals[:-1] + vals[1:]) / 2.0
    pts = np.concatenate([vals, mids, [448.0, 456.0, 464.0, 472.0, 480.0, 1e4, 3.0e38,
                                       2.0 ** -10, 2.0 ** -11, 2.0 ** -12]])
    pts32 = pts.astype(np.float32)
    up = np.nextafter(pts32, np.float32(np.inf))
    dn = np.nextafter(pts32, np.float32(0))
    allp = np.concatenate([pts32, up, dn, np.array([0.0, 1e-45, 1e-38], np.float32)])
    allp = np.unique(allp[np.isfinite(allp)])
    return np.concatenate([allp, -allp]).astype(np.float32)


def check_decode(decode_fn, golden_rows):
    """decode agrees with the format table and with the library on all codes."""
    got = decode_fn(np.arange(256, dtype=np.uint8))
    lib = torch_decode_all()
    same = (got == lib) | (np.isnan(got) & np.isnan(lib))
    assert same.all(), np.nonzero(~same)
    # signed zero
    assert np.signbit(got[0x80]) and not np.signbit(got[0x00])
    for code, val in golden_rows:
        g = decode_fn(np.array([code], dtype=np.uint8))[0]
        if np.isnan(val):
            assert np.isnan(g), (hex(code), g)
        else:
            assert g == val and np.signbit(g) == np.signbit(val), (hex(code), g, val)


def check_encode_points(encode_fn, pts):
    got = encode_fn(pts)
    bf = bruteforce_encode(pts)
    lib = library_encode(pts)
    assert (bf == lib).all(), "brute force and library disagree"
    bad = np.nonzero(got != bf)[0]
    assert bad.size == 0, [(float(pts[i]), int(got[i]), int(bf[i])) for i in bad[:10]]


def check_encode_binade(encode_fn, exp_field):
    """Every float32 with the given biased exponent field, positive sign:
    equal to the library cast, and monotone non-decreasing in value."""
    bits = np.arange(1 << 23, dtype=np.uint32) | np.uint32(exp_field << 23)
    x = bits.view(np.float32)
    got = encode_fn(x)
    lib = library_encode(x)
    bad = np.nonzero(got != lib)[0]
    assert bad.size == 0, [(float(x[i]), int(got[i]), int(lib[i])) for i in bad[:10]]
    assert (np.diff(got.astype(np.int32)) >= 0).all()
    return got[0], got[-1]


# ---------------------------------------------------------------- quantiser

def check_amax_maps_to_448(quant_group_fn, rng, n=200):
    """Every non-zero group contains +-448 (code 0x7E or 0xFE)."""
    for _ in range(n):
        scale = np.float32(2.0 ** rng.integers(-30, 30))
        x = (rng.standard_normal(GROUP) * scale).astype(np.float32)
        q, s = quant_group_fn(x)
        assert np.any((q == 0x7E) | (q == 0xFE)), (x, q, s)


def check_scale_invariance(quant_group_fn, rng, n=100):
    """Scaling a group by 2**j leaves the codes alone and scales s by 2**j."""
    for _ in range(n):
        x = (rng.standard_normal(GROUP) * np.exp(rng.standard_normal())).astype(np.float32)
        q0, s0 = quant_group_fn(x)
        for j in (-20, -7, -1, 1, 5, 20):
            f = np.float32(2.0 ** j)
            q1, s1 = quant_group_fn((x * f).astype(np.float32))
            assert (q1 == q0).all(), j
            assert np.float32(s1) == np.float32(s0 * f), (j, s0, s1)


def check_exact_representability(quant_group_fn, decode_vals, rng, n=100):
    """A group of E4M3 values times 2**j containing +-448*2**j round-trips
    exactly and gets the scale 2**j."""
    finite = decode_vals[:127]
    for _ in range(n):
        j = int(rng.integers(-40, 40))
        v = rng.choice(finite, GROUP) * rng.choice([-1.0, 1.0], GROUP)
        v[int(rng.integers(GROUP))] = 448.0 * rng.choice([-1.0, 1.0])
        x = (v * 2.0 ** j).astype(np.float32)
        q, s = quant_group_fn(x)
        assert np.float32(s) == np.float32(2.0 ** j), (j, s)
        back = torch_decode_all()[q] * np.float64(s)
        assert (back == x.astype(np.float64)).all()


def check_roundtrip_bound(quant_group_fn, rng, n=200):
    """|dec(q)*s - x| <= (2**-4 + 2**-20)|x| where |x*inv| is in the normal
    range, and <= 2**-10 s + 2**-20 |x| otherwise."""
    for _ in range(n):
        x = (rng.standard_t(3, GROUP) * 2.0 ** rng.integers(-20, 20)).astype(np.float32)
        q, s = quant_group_fn(x)
        back = torch_decode_all()[q] * np.float64(s)
        xd = x.astype(np.float64)
        err = np.abs(back - xd)
        y = np.abs(xd) / np.float64(s)
        normal = y >= 2.0 ** -6
        bound = np.where(normal, (2.0 ** -4 + 2.0 ** -20) * np.abs(xd),
                         2.0 ** -10 * np.float64(s) + 2.0 ** -20 * np.abs(xd))
        assert (err <= bound).all(), np.max(err / np.maximum(bound, 1e-300))


def check_zero_group(quant_group_fn):
    x = np.zeros(GROUP, np.float32)
    x[::3] = -0.0
    q, s = quant_group_fn(x)
    assert np.float32(s) == np.float32(1.0)
    assert ((q == 0x00) | (q == 0x80)).all()
    assert (q[::3] == 0x80).all() and (q[1::3] == 0x00).all()


# ---------------------------------------------------------------- GEMM

def _lib_dec(q):
    return torch_decode_all()[np.asarray(q, np.uint8)]


def integer_exact_operands(rng, layout, mode_a, mode_b, M, N, K):
    """Codes that decode to integers in [-8, 8] and power-of-two scales.

    Returns stored operands (qa, sa, qb, sb) per the layout letters.  With
    K <= 1024 every partial sum, promotion and total is exact in float32.
    """
    int_codes = np.array([c for c in range(256) if np.isfinite(_lib_dec(c))
                          and float(_lib_dec(c)).is_integer() and abs(_lib_dec(c)) <= 8],
                         dtype=np.uint8)

    def stored(role, trans, mode):
        if role == "A":
            shape = (M, K) if trans == "N" else (K, M)
            k_axis = 1 if trans == "N" else 0
        else:
            shape = (K, N) if trans == "N" else (N, K)
            k_axis = 0 if trans == "N" else 1
        q = rng.choice(int_codes, shape).astype(np.uint8)
        if mode == "act":
            sshape = list(shape)
            sshape[k_axis] //= GROUP
        else:
            sshape = [shape[0] // GROUP, shape[1] // GROUP]
        s = (2.0 ** rng.integers(-3, 4, tuple(sshape))).astype(np.float32)
        return q, s

    qa, sa = stored("A", layout[0], mode_a)
    qb, sb = stored("B", layout[1], mode_b)
    return qa, sa, qb, sb


def exact_gemm_int(layout, qa, sa, mode_a, qb, sb, mode_b):
    """Exact product for integer-valued codes and power-of-two scales.

    Builds each logical element as an integer times a power of two by
    explicit per-element loops over the K blocks (int64 matmul per block,
    then exact float64 scaling), independent of the oracle's dequantiser.
    """
    A = _lib_dec(qa).astype(np.int64)
    B = _lib_dec(qb).astype(np.int64)
    A = A if layout[0] == "N" else A.T  # logical [M][K]
    B = B if layout[1] == "N" else B.T  # logical [K][N]
    M, K = A.shape
    N = B.shape[1]

    def scale_a(kb):  # -> [M]
        if mode_a == "act":
            return sa[:, kb] if layout[0] == "N" else sa[kb, :]
        rows = np.arange(M) // GROUP
        return sa[rows, kb] if layout[0] == "N" else sa[kb, rows]

    def scale_b(kb):  # -> [N]
        if mode_b == "act":
            return sb[kb, :] if layout[1] == "N" else sb[:, kb]
        cols = np.arange(N) // GROUP
        return sb[kb, cols] if layout[1] == "N" else sb[cols, kb]

    R = np.zeros((M, N), np.float64)
    for kb in range(K // GROUP):
        sl = slice(kb * GROUP, (kb + 1) * GROUP)
        P = A[:, sl] @ B[sl, :]  # exact int64
        R += P.astype(np.float64) * scale_a(kb).astype(np.float64)[:, None] \
            * scale_b(kb).astype(np.float64)[None, :]
    return R


def fraction_gemm(layout, qa, sa, mode_a, qb, sb, mode_b):
    """Brute-force exact rational sum over every (m, n, k); tiny shapes only."""
    A = _lib_dec(qa)
    B = _lib_dec(qb)
    A = A if layout[0] == "N" else A.T
    B = B if layout[1] == "N" else B.T
    M, K = A.shape
    N = B.shape[1]

    def sA(m, k):
        kb = k // GROUP
        if mode_a == "act":
            return sa[m, kb] if layout[0] == "N" else sa[kb, m]
        return sa[m // GROUP, kb] if layout[0] == "N" else sa[kb, m // GROUP]

    def sB(k, n):
        kb = k // GROUP
        if mode_b == "act":
            return sb[kb, n] if layout[1] == "N" else sb[n, kb]
        return sb[kb, n // GROUP] if layout[1] == "N" else sb[n // GROUP, kb]

    out = np.zeros((M, N), np.float64)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += (Fraction(float(A[m, k])) * Fraction(float(sA(m, k)))
                        * Fraction(float(B[k, n])) * Fraction(float(sB(k, n))))
            out[m, n] = float(acc)
    return out


def fraction_gemm_points(layout, qa, sa, mode_a, qb, sb, mode_b, rows, cols):
    """Exact rational sums for selected output rows x cols only."""
    A = _lib_dec(qa)
    B = _lib_dec(qb)
    A = A if layout[0] == "N" else A.T
    B = B if layout[1] == "N" else B.T
    K = A.shape[1]

    def sA(m, k):
        kb = k // GROUP
        if mode_a == "act":
            return sa[m, kb] if layout[0] == "N" else sa[kb, m]
        return sa[m // GROUP, kb] if layout[0] == "N" else sa[kb, m // GROUP]

    def sB(k, n):
        kb = k // GROUP
        if mode_b == "act":
            return sb[kb, n] if layout[1] == "N" else sb[n, kb]
        return sb[kb, n // GROUP] if layout[1] == "N" else sb[n // GROUP, kb]

    out = np.zeros((len(rows), len(cols)), np.float64)
    for i, m in enumerate(rows):
        for j, n in enumerate(cols):
            acc = Fraction(0)
            for k in range(K):
                acc += (Fraction(float(A[m, k])) * Fraction(float(sA(m, k)))
                        * Fraction(float(B[k, n])) * Fraction(float(sB(k, n))))
            out[i, j] = float(acc)
    return out
