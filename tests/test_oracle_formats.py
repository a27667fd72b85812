"""Pins of the oracle's code tables and element rounding (CPU only).

Each test checks the oracle against something other than itself: hand-derived
fixtures under tests/golden/, torch's float8_e4m3fn conversion, or a brute
force nearest-value search in exact rational arithmetic.
"""

from fractions import Fraction
import math

import numpy as np
import pytest
import torch

import oracle
from conftest import golden_lines


def all_finite_bf16_bits():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    return bits[exp != 0xFF]


# --------------------------------------------------------------- E2M1 -----

def test_e2m1_decode_matches_golden_table():
    rows = list(golden_lines("e2m1_codes.txt"))
    assert len(rows) == 16
    codes = np.array([int(c, 16) for c, _ in rows], dtype=np.uint8)
    want = np.array([float(v) for _, v in rows])
    got = oracle.e2m1_decode(codes)
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))  # -0 for 0x8


def test_e2m1_magnitudes_are_the_fp4_value_set():
    assert list(oracle.E2M1_MAGNITUDES) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def test_e2m1_rounding_golden_ties_and_saturation():
    for r, code in golden_lines("e2m1_rounding.txt"):
        got = int(oracle.e2m1_encode(np.array([float(r)]))[0])
        assert got == int(code, 16), (r, hex(got), code)


def _fraction_nearest_e2m1(r):
    """Brute force: nearest signed E2M1 value in exact rationals, even code on ties."""
    best = None
    for code in range(16):
        sign = -1 if code & 8 else 1
        mag = Fraction(oracle.E2M1_MAGNITUDES[code & 7]).limit_denominator()
        if (sign < 0) != (r < 0 or (r == 0 and math.copysign(1, r) < 0)):
            continue
        d = abs(r - sign * mag)
        key = (d, code & 1)  # smaller distance first, then even mantissa bit
        if best is None or key < best[0]:
            best = (key, code)
    return best[1]


def test_e2m1_encode_vs_exact_bruteforce_sampled():
    g = np.random.default_rng(1234)
    # random magnitudes around the grid, exact midpoints and huge/tiny values
    r = np.concatenate([
        g.uniform(-9, 9, 3000),
        np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]) * g.choice([-1, 1], 7),
        np.ldexp(g.uniform(1, 2, 200), g.integers(-140, 10, 200)) * g.choice([-1, 1], 200),
    ])
    got = oracle.e2m1_encode(r)
    for x, c in zip(r, got):
        assert int(c) == _fraction_nearest_e2m1(Fraction(float(x))), x


def test_e2m1_encode_exhaustive_bf16_against_float_argmin():
    """Every finite bf16 value times every power of two 2^-E, E in [-127, 127].

    The reference is an argmin over the 8 grid magnitudes computed in float64
    (exact here: every value is a short dyadic rational) with the even code
    winning ties, which is independent of the oracle's binade arithmetic.
    """
    bits = all_finite_bf16_bits()
    v = oracle.bf16_bits_to_f64(bits)
    grid = oracle.E2M1_MAGNITUDES
    for e in range(-127, 128, 1):
        r = v / np.ldexp(1.0, e)
        # every |r| >= 6 has 6 as its nearest grid value; clamping keeps the
        # float64 distances exact (no absorption against huge magnitudes)
        a = np.minimum(np.abs(r), 8.0)
        d = np.abs(a[:, None] - grid[None, :])
        dmin = d.min(axis=1, keepdims=True)
        cand = d == dmin
        # among the nearest magnitudes prefer an even code
        even = cand & (np.arange(8)[None, :] % 2 == 0)
        pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
        want = pick | (np.signbit(r).astype(np.int64) << 3)
        got = oracle.e2m1_encode(r).astype(np.int64)
        assert np.array_equal(got, want), e


# -------------------------------------------------------------- E4M3FN ----

def test_e4m3fn_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3fn_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))


def test_e4m3fn_golden_points():
    for row in golden_lines("e4m3fn_points.txt"):
        kind, a, b = row
        if kind == "decode":
            got = float(oracle.e4m3fn_decode(np.array([int(a, 16)], np.uint8))[0])
            if b == "nan":
                assert math.isnan(got)
            else:
                assert got == float(b) and math.copysign(1, got) == math.copysign(1, float(b)), row
        else:
            got = int(oracle.e4m3fn_encode(np.array([float(a)]))[0])
            assert got == int(b, 16), (row, hex(got))


def test_e4m3fn_encode_matches_torch_cast_within_range():
    """torch's float32 -> float8_e4m3fn cast is RNE (it returns NaN only above 464)."""
    g = np.random.default_rng(7)
    x = np.concatenate([
        g.uniform(-448, 448, 20000),
        np.ldexp(g.uniform(1, 2, 20000), g.integers(-14, 9, 20000)) * g.choice([-1, 1], 20000),
        # exact midpoints between neighbouring codes
        (oracle.e4m3fn_decode(np.arange(0x7E, dtype=np.uint8))
         + oracle.e4m3fn_decode(np.arange(1, 0x7F, dtype=np.uint8))) / 2,
    ]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3fn_encode(x.astype(np.float64))
    assert np.array_equal(got, want)


def test_e4m3fn_saturates_instead_of_nan():
    got = oracle.e4m3fn_encode(np.array([465.0, 1000.0, 3e38, -500.0]))
    assert list(got) == [0x7E, 0x7E, 0x7E, 0xFE]


# ---------------------------------------------------------------- E8M0 ----

def test_e8m0_decode_closed_form():
    got = oracle.e8m0_decode(np.array([0, 1, 126, 127, 128, 254, 255], np.uint8))
    assert got[0] == 2.0 ** -127 and got[1] == 2.0 ** -126
    assert got[2] == 0.5 and got[3] == 1.0 and got[4] == 2.0
    assert got[5] == 2.0 ** 127 and math.isnan(got[6])


def test_bf16_bits_roundtrip_through_torch():
    bits = all_finite_bf16_bits()
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_bits_to_f64(bits)
    assert np.array_equal(got, want)


def test_f64_to_bf16_matches_torch_rne_on_fp32_inputs():
    """bf16 output rounding against torch's fp32 -> bf16 conversion (IEEE RNE).

    Inputs are fp32-representable so that torch rounds once: every exact
    midpoint between neighbouring bf16 values (ties, low half 0x8000), the
    values one fp32 ulp either side of it, subnormals, and the overflow edge.
    """
    g = np.random.default_rng(7)
    hi = g.integers(0, 1 << 16, size=200_000, dtype=np.uint32)
    hi = hi[(hi & 0x7F80) != 0x7F80]  # finite bf16 prefixes
    low = np.array([0x0000, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x1234], np.uint32)
    u = ((hi[:, None] << np.uint32(16)) | low[None, :]).ravel()
    x32 = u.view(np.float32)
    want = torch.from_numpy(x32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f64_to_bf16_bits(x32.astype(np.float64))
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, (u[bad[:4]], got[bad[:4]], want[bad[:4]])


def test_f64_to_bf16_closed_forms():
    f = lambda v: int(oracle.f64_to_bf16_bits(np.array([v]))[0])
    assert f(1.0) == 0x3F80 and f(-2.0) == 0xC000 and f(-0.0) == 0x8000
    assert f(1.0 + 2.0 ** -8) == 0x3F80          # tie -> even (1.0)
    assert f(1.0 + 3 * 2.0 ** -8) == 0x3F82      # tie -> even (1 + 2^-6)
    assert f(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81  # just above the tie (not fp32-representable)
    assert f(2.0 ** -133) == 0x0001 and f(2.0 ** -134) == 0x0000  # smallest subnormal; tie to zero
    assert f(oracle.BF16_MAX) == 0x7F7F
    assert f(oracle.BF16_MAX + 2.0 ** 119) == 0x7F80  # halfway to 2^128 -> even -> inf
    assert f(-1e300) == 0xFF80
