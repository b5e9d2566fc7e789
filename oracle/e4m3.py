"""OCP E4M3 ("E4M3FN") codec, written out from the format's definition.

Source of the definition: FP8 Formats for Deep Learning (Micikevicius et al.,
2022), the E4M3 row of its format table; the Puro-2B paper translation
(papers.lianghsun.dev) cites it in its reference list and, in section 3.2,
names E4M3 as the operand format of every Transformer linear layer.

Format: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits.
  * exponent field 0: subnormal, value = m * 2**-9
  * otherwise:        value = (1 + m/8) * 2**(E - 7)
  * S.1111.111 is NaN; there are no infinities; largest finite is 0x7E = 448.

Encoding is saturating round-to-nearest-even (a reading: the pages name the
format but not the rounding).  All arithmetic below is done
in float64 on values that are exactly representable there, so every step is
exact except the one rounding the definition asks for (numpy.rint, which
rounds halves to even).
"""

import numpy as np

E4M3_MAX = 448.0
_MIN_NORMAL = 2.0 ** -6  # code 0x08
_SUBNORMAL_STEP = 2.0 ** -9  # code 0x01


def e4m3_decode(codes):
    """Decode uint8 E4M3 codes to float64 (NaN for S.1111.111).

    Follows the definition in the module docstring term by term.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c & 0x80) != 0, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    sub = m * _SUBNORMAL_STEP
    nrm = (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64))
    mag = np.where(e == 0, sub, nrm)
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(y):
    """Encode float32 values to E4M3 codes, saturating, round-half-to-even.

    Steps, for a = |y|:
      1. a >= 448           -> 0x7E (saturate; 448 itself is exact)
      2. a <  2**-6         -> n = RNE(a * 2**9) in [0, 8]; code n
                               (n == 8 is the smallest normal, code 0x08)
      3. otherwise e = floor(log2 a) in [-6, 8]; n = RNE(a * 2**(3-e)) in
         [8, 16]; n == 16 carries into the exponent; code ((e+7)<<3)|(n-8)
      4. OR in the sign bit (so -0 and negative values that round to zero
         give 0x80).
    Non-finite inputs are outside the contract (no NaN is ever produced for
    a finite input); NaN input maps to 0x7F with its sign for completeness.
    """
    y32 = np.asarray(y, dtype=np.float32)
    a = np.abs(y32.astype(np.float64))
    neg = np.signbit(y32)

    code = np.zeros(a.shape, dtype=np.int64)

    # step 2: subnormal range (and zero)
    small = a < _MIN_NORMAL
    n_sub = np.rint(a * 2.0 ** 9).astype(np.int64)
    code = np.where(small, n_sub, code)

    # step 3: normal range below the saturation point
    normal = (~small) & (a < E4M3_MAX)
    a_safe = np.where(normal, a, 1.0)
    _, ex = np.frexp(a_safe)  # a = f * 2**ex, f in [0.5, 1)
    e = ex.astype(np.int64) - 1  # floor(log2 a)
    n = np.rint(a_safe * np.exp2((3 - e).astype(np.float64))).astype(np.int64)
    carry = n == 16
    e = np.where(carry, e + 1, e)
    n = np.where(carry, 8, n)
    code_n = ((e + 7) << 3) | (n - 8)
    code = np.where(normal, code_n, code)

    # step 1: saturation
    code = np.where(a >= E4M3_MAX, 0x7E, code)

    nan = np.isnan(y32)
    code = np.where(nan, 0x7F, code)

    code = code | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)
