"""Pins for the oracle's E4M3 codec (CPU only).

Decode: the format table of FP8 Formats for Deep Learning (golden fixture)
and the library decode of torch.float8_e4m3fn on all 256 codes.
Encode: brute-force nearest search and the library cast at every rounding
decision point, and the library cast exhaustively over every positive
float32 in [2**-11, 2**10) (every binade where rounding happens), plus
monotonicity, sign symmetry and the saturated/underflow tails.
"""
import os

import numpy as np
import pytest

import pins
from oracle import e4m3_decode, e4m3_encode

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_format_table.txt")


def golden_rows():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        code, val, _name = line.split()
        rows.append((int(code, 16), float(val)))
    return rows


def test_decode_table_and_library():
    pins.check_decode(e4m3_decode, golden_rows())


def test_encode_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert (e4m3_encode(e4m3_decode(codes).astype(np.float32)) == codes).all()


def test_encode_critical_points_vs_bruteforce_and_library():
    pins.check_encode_points(e4m3_encode, pins.critical_points())


def test_encode_random_vs_bruteforce():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(20000) * 2.0 ** rng.integers(-12, 10, 20000)).astype(np.float32)
    pins.check_encode_points(e4m3_encode, x)


def test_encode_exhaustive_rounding_binades():
    # biased float32 exponent 116 is 2**-11 ... 136 is 2**9 (up to 2**10)
    prev_last = 0
    for ef in range(116, 137):
        first, last = pins.check_encode_binade(e4m3_encode, ef)
        assert first >= prev_last  # monotone across binade boundaries too
        prev_last = last
    assert prev_last == 0x7E


def test_encode_sign_symmetry_and_tails():
    rng = np.random.default_rng(2)
    bits = rng.integers(0, 0x7F800000, 200000, dtype=np.uint32)
    x = bits.view(np.float32)
    pos = e4m3_encode(x)
    neg = e4m3_encode(-x)
    assert (neg == (pos | 0x80)).all()
    # below 2**-11 everything is a (signed) zero; from 2**10 up it saturates
    small = x[x < 2.0 ** -11]
    assert (e4m3_encode(small) == 0).all() and (e4m3_encode(-small) == 0x80).all()
    big = x[x >= 2.0 ** 10]
    assert (e4m3_encode(big) == 0x7E).all() and (e4m3_encode(-big) == 0xFE).all()
    assert (pins.library_encode(big) == 0x7E).all()


def test_saturation_tie_and_library_nan_difference():
    # 464 is the midpoint of 448 and the (absent) 480: RNE keeps 448.
    x = np.array([448.0, 456.0, 464.0, 470.0, 479.0, 1e30], np.float32)
    assert (e4m3_encode(x) == 0x7E).all()
    # the unclamped library cast does not saturate (470 -> NaN); the oracle does
    import torch
    raw = torch.tensor([470.0]).to(torch.float8_e4m3fn).view(torch.uint8).item()
    assert raw == 0x7F
