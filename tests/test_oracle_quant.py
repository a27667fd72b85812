"""Pins of the oracle's MXFP4 and FP8 per-token quantizers (CPU only)."""

from fractions import Fraction
import math

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
from conftest import golden_lines


def _floor_log2_fraction(q):
    """floor(log2 q) of a positive Fraction, by integer bit lengths."""
    n, d = q.numerator, q.denominator
    e = n.bit_length() - d.bit_length()
    # now 2^(e-1) < n/d < 2^(e+1); settle the boundary exactly
    if Fraction(n, d) < Fraction(2) ** e:
        e -= 1
    return e


# ------------------------------------------------------- shared exponent ----

def test_scale_exponent_exhaustive_over_bf16():
    bits = np.arange(1, 0x7F80, dtype=np.uint32).astype(np.uint16)  # every positive finite bf16
    amax = oracle.bf16_bits_to_f64(bits)
    got = oracle.mxfp4_scale_exponent(amax)
    for b, a, e in zip(bits[::7], amax[::7], got[::7]):
        want = max(-127, min(127, _floor_log2_fraction(Fraction(float(a))) - 2))
        assert e == want, (hex(b), a, e, want)
    # the full set against the bf16 exponent field: floor(log2) = field - 127 for normals
    field = (bits >> 7).astype(np.int64)
    normal = field > 0
    assert np.array_equal(got[normal], np.clip(field[normal] - 129, -127, 127))
    assert np.all(got[~normal] == -127)  # subnormal bf16 blocks clamp to 2^-127
    assert oracle.mxfp4_scale_exponent(np.array([0.0]))[0] == -127


def test_block_amax_lands_in_4_to_8():
    g = np.random.default_rng(3)
    x = (g.standard_normal((64, 256)) * np.ldexp(1.0, g.integers(-60, 60, (64, 1)))).astype(np.float32)
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    _, scales = oracle.mxfp4_quantize(bits)
    v = oracle.bf16_bits_to_f64(bits).reshape(64, 8, 32)
    amax = np.abs(v).max(axis=2)
    ratio = amax / np.ldexp(1.0, scales.astype(np.int64) - 127)
    assert np.all((ratio >= 4) & (ratio < 8))


# --------------------------------------------------------- MXFP4 golden ----

def _read_mxfp4_row():
    blocks, packed = {}, {}
    cur = None
    for row in golden_lines("mxfp4_row.txt"):
        if row[0] == "block":
            cur = int(row[1])
            blocks[cur] = {"scale": int(row[3]), "elems": []}
        elif row[0] == "packed":
            packed[int(row[1])] = bytes(int(b, 16) for b in row[2:])
        else:
            blocks[cur]["elems"].append((int(row[0]), int(row[1], 16), int(row[2], 16)))
    return blocks, packed


def test_mxfp4_golden_row():
    blocks, packed = _read_mxfp4_row()
    nb = len(blocks)
    x = np.zeros((1, 32 * nb), dtype=np.uint16)
    for j, blk in blocks.items():
        for pos, b, _ in blk["elems"]:
            x[0, 32 * j + pos] = b
    codes, scales = oracle.mxfp4_quantize(x)
    assert list(scales[0]) == [blocks[j]["scale"] for j in range(nb)]
    nib = oracle.unpack_nibbles(codes)[0]
    for j, blk in blocks.items():
        want = np.zeros(32, np.uint8)
        for pos, _, c in blk["elems"]:
            want[pos] = c
        assert np.array_equal(nib[32 * j: 32 * j + 32], want), j
        assert bytes(codes[0, 16 * j: 16 * j + 16]) == packed[j], j


def _fraction_quantize_block(vals):
    """Independent scalar MXFP4 quantizer for one block, in exact rationals."""
    fr = [Fraction(float(v)) for v in vals]
    amax = max(abs(f) for f in fr)
    e = -127 if amax == 0 else max(-127, min(127, _floor_log2_fraction(amax) - 2))
    scale = Fraction(2) ** e
    grid = [Fraction(int(2 * m), 2) for m in oracle.E2M1_MAGNITUDES]
    codes = []
    for f, v in zip(fr, vals):
        r = f / scale
        mags = sorted(range(8), key=lambda c: (abs(abs(r) - grid[c]), c & 1))
        codes.append(mags[0] | (8 if math.copysign(1.0, float(v)) < 0 else 0))
    return e + 127, codes


def test_mxfp4_vs_exact_scalar_quantizer_random_blocks():
    g = np.random.default_rng(11)
    raw = g.standard_t(3, (40, 64)).astype(np.float32) * np.ldexp(1.0, g.integers(-130, 120, (40, 1)))
    raw[3, :32] = 0.0
    raw[4, 5] = -0.0
    bits = torch.from_numpy(raw.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    codes, scales = oracle.mxfp4_quantize(bits)
    nib = oracle.unpack_nibbles(codes)
    v = oracle.bf16_bits_to_f64(bits)
    for i in range(bits.shape[0]):
        for j in range(2):
            s, c = _fraction_quantize_block(v[i, 32 * j: 32 * j + 32])
            assert scales[i, j] == s, (i, j)
            assert list(nib[i, 32 * j: 32 * j + 32]) == c, (i, j)


def _bits_from_f64(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@settings(max_examples=150, deadline=None)
@given(st.lists(st.integers(0, 15), min_size=32, max_size=32), st.integers(-120, 120))
def test_mxfp4_roundtrip_of_representable_blocks(codes, e):
    """A block of E2M1 values times 2^e re-quantizes to the same values."""
    vals = oracle.e2m1_decode(np.array(codes, np.uint8)) * np.ldexp(1.0, e)
    bits = _bits_from_f64(vals[None, :])
    q, s = oracle.mxfp4_quantize(bits)
    back = oracle.mxfp4_dequantize(q, s)[0]
    assert np.array_equal(back, vals)


@settings(max_examples=150, deadline=None)
@given(st.lists(st.floats(-1e4, 1e4, allow_nan=False, width=32), min_size=64, max_size=64),
       st.integers(-100, 100))
def test_mxfp4_idempotent(vals, e):
    """Q(DQ(Q(x))) == Q(x) byte for byte."""
    bits = _bits_from_f64(np.array(vals) * 2.0 ** e)[None, :]
    q1, s1 = oracle.mxfp4_quantize(bits)
    dq = oracle.mxfp4_dequantize(q1, s1)
    q2, s2 = oracle.mxfp4_quantize(_bits_from_f64(dq))
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


def test_mxfp4_sign_symmetry_and_scale_invariance():
    g = np.random.default_rng(5)
    bits = _bits_from_f64(g.standard_normal((16, 128)))
    q, s = oracle.mxfp4_quantize(bits)
    qn, sn = oracle.mxfp4_quantize(bits ^ np.uint16(0x8000))
    assert np.array_equal(sn, s)
    assert np.array_equal(oracle.unpack_nibbles(qn), oracle.unpack_nibbles(q) ^ 8)
    # multiplying by 2^k shifts every scale by k and leaves the codes alone
    q3, s3 = oracle.mxfp4_quantize(_bits_from_f64(oracle.bf16_bits_to_f64(bits) * 8.0))
    assert np.array_equal(q3, q) and np.array_equal(s3.astype(int), s.astype(int) + 3)


# ------------------------------------------------------------------ FP8 ----

def test_fp8_golden_rows():
    rows, cur = {}, None
    for row in golden_lines("fp8_rows.txt"):
        if row[0] == "row":
            cur = int(row[1])
            rows[cur] = {"scale": float(row[3]), "elems": []}
        else:
            rows[cur]["elems"].append((int(row[0]), int(row[1], 16), int(row[2], 16)))
    x = np.zeros((len(rows), 32), np.uint16)
    for i, r in rows.items():
        for pos, b, _ in r["elems"]:
            x[i, pos] = b
    codes, scales = oracle.fp8_quantize_per_token(x)
    for i, r in rows.items():
        assert scales[i] == np.float32(r["scale"]), i
        want = np.zeros(32, np.uint8)
        for pos, _, c in r["elems"]:
            want[pos] = c
        assert np.array_equal(codes[i], want), (i, codes[i])


def test_fp8_matches_torch_division_and_cast():
    """Independent route: torch fp32 amax / 448, torch fp32 division, torch E4M3FN cast."""
    g = np.random.default_rng(21)
    x = g.standard_normal((64, 512)).astype(np.float32) * np.ldexp(1.0, g.integers(-40, 40, (64, 1))).astype(np.float32)
    x[:, 17] *= 30
    bits = _bits_from_f64(x)
    codes, scales = oracle.fp8_quantize_per_token(bits)
    xt = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32)
    st_ = xt.abs().amax(dim=1) / torch.tensor(448.0, dtype=torch.float32)
    q = xt / st_[:, None]
    want = q.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(scales, st_.numpy())
    assert np.array_equal(codes, want)


def test_fp8_scale_is_correctly_rounded_quotient():
    g = np.random.default_rng(8)
    amax = np.ldexp(g.uniform(1, 2, 5000), g.integers(-133, 127, 5000)).astype(np.float32)
    amax = amax[np.isfinite(amax) & (amax > 0)]
    x = np.zeros((len(amax), 32), np.float32)
    x[:, 0] = amax
    bits = _bits_from_f64(x)
    _, s = oracle.fp8_quantize_per_token(bits)
    a32 = oracle.bf16_bits_to_f32(bits[:, 0])
    for a, si in zip(a32[::5], s[::5]):
        exact = Fraction(float(a)) / 448
        # correct rounding: no other float32 lies closer to the exact quotient
        up = np.nextafter(si, np.float32(np.inf))
        dn = np.nextafter(si, np.float32(0))
        err = abs(Fraction(float(si)) - exact)
        assert err <= abs(Fraction(float(up)) - exact) and err <= abs(Fraction(float(dn)) - exact)


def test_fp8_row_amax_maps_to_448_and_zero_row():
    g = np.random.default_rng(4)
    bits = _bits_from_f64(g.standard_normal((50, 320)) * 3)
    codes, s = oracle.fp8_quantize_per_token(bits)
    assert np.all((codes & 0x7F).max(axis=1) == 0x7E)
    zero = np.zeros((2, 64), np.uint16)
    zero[1, 3] = 0x8000
    zc, zs = oracle.fp8_quantize_per_token(zero)
    assert np.all(zs == 0) and zc[1, 3] == 0x80 and np.count_nonzero(zc) == 1


def test_fp8_dequantize_closed_form():
    codes = np.array([[0x38, 0xB8, 0x7E, 0x01]], np.uint8)
    got = oracle.fp8_dequantize_per_token(codes, np.array([0.5], np.float32))
    assert list(got[0]) == [0.5, -0.5, 224.0, 2.0 ** -10]


def test_fp8_quotient_is_correctly_rounded_division():
    """The fp32 quotient is x / s rounded once (not x times a rounded reciprocal)."""
    g = np.random.default_rng(17)
    x = (g.standard_normal((40, 64)) * np.ldexp(1.0, g.integers(-30, 30, (40, 1)))).astype(np.float32)
    x32 = oracle.bf16_bits_to_f32(_bits_from_f64(x))
    s = oracle.fp8_per_token_scale(x32)
    r = oracle.fp8_scaled_quotient(x32, s)
    recip_differs = 0
    for i in range(0, 40, 3):
        for j in range(64):
            exact = Fraction(float(x32[i, j])) / Fraction(float(s[i]))
            q = r[i, j]
            err = abs(Fraction(float(q)) - exact)
            for nb in (np.nextafter(q, np.float32(np.inf)), np.nextafter(q, np.float32(-np.inf))):
                assert err <= abs(Fraction(float(nb)) - exact), (i, j)
            recip_differs += int(np.float32(x32[i, j] * (np.float32(1) / s[i])) != q)
    assert recip_differs > 0  # the sample does separate the two forms


# ----------------------------------------------------------- FP8 static ----

def _static_golden():
    groups, cur = [], None
    for row in golden_lines("fp8_static.txt"):
        if row[0] == "amax":
            cur = {"amax": int(row[1], 16), "scale": None if row[3] == "-" else float(row[3]), "elems": []}
            groups.append(cur)
        else:
            cur["elems"].append((int(row[0], 16), int(row[1], 16)))
    return groups


def test_fp8_static_golden():
    groups = _static_golden()
    assert len(groups) == 6
    for gr in groups:
        amax = oracle.bf16_bits_to_f32(np.array([gr["amax"]], np.uint16))[0]
        x = np.zeros((1, 32), np.uint16)
        for i, (b, _) in enumerate(gr["elems"]):
            x[0, i] = b
        codes, scales = oracle.fp8_quantize_static(x, amax)
        if gr["scale"] is not None:
            assert scales[0] == np.float32(gr["scale"])
        for i, (b, c) in enumerate(gr["elems"]):
            assert codes[0, i] == c, (hex(gr["amax"]), hex(b), hex(codes[0, i]), hex(c))


def test_fp8_static_equals_per_token_when_every_row_has_the_amax():
    """Rows whose own amax is the calibrated one: the static rule is the per-token rule."""
    g = np.random.default_rng(31)
    x = g.standard_normal((40, 256)) * 2.0
    x[:, 0] = 9.0
    x[1::2, 0] = -9.0  # the amax may come with either sign
    bits = _bits_from_f64(np.clip(x, -9.0, 9.0))
    c_tok, s_tok = oracle.fp8_quantize_per_token(bits)
    c_st, s_st = oracle.fp8_quantize_static(bits, np.float32(9.0))
    assert np.array_equal(s_tok, s_st) and np.array_equal(c_tok, c_st)


def test_fp8_static_matches_torch_below_saturation():
    """Independent route: torch fp32 division and torch's E4M3FN cast where |x / s| < 464,
    and the saturated code where it is not (torch's cast turns those into NaN)."""
    g = np.random.default_rng(32)
    x = (g.standard_normal((48, 512)) * np.ldexp(1.0, g.integers(-20, 20, (48, 1)))).astype(np.float32)
    bits = _bits_from_f64(x)
    xt = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32)
    for frac in (1.0, 0.3, 1e-3, 7.5):
        amax = np.float32(float(xt.abs().max()) * frac)
        codes, scales = oracle.fp8_quantize_static(bits, amax)
        s = torch.tensor(amax, dtype=torch.float32) / torch.tensor(448.0, dtype=torch.float32)
        assert np.all(scales == s.numpy())
        q = xt / s
        small = q.abs() < 464
        want = q.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        sat = np.where(np.signbit(q.numpy()), 0xFE, 0x7E).astype(np.uint8)
        want = np.where(small.numpy(), want, sat)
        assert np.array_equal(codes, want), frac
        if frac < 1:
            assert np.count_nonzero(~small.numpy()) > 0  # saturation is exercised


def test_fp8_static_monotone_and_saturating_over_all_bf16():
    """Over every finite bf16 x (one amax), the decoded code is a non-decreasing
    function of x, odd, at most 448, and 448 exactly from x / s >= 432 on."""
    pos = np.arange(0, 0x7F80, dtype=np.uint32).astype(np.uint16)
    bits = np.concatenate([pos, pos | 0x8000]).reshape(-1, 32)
    amax = np.float32(3.296875)  # a bf16 value that is no power of two
    codes, s = oracle.fp8_quantize_static(bits, amax)
    codes = codes.reshape(-1)
    x = oracle.bf16_bits_to_f64(bits.reshape(-1))
    v = oracle.e4m3fn_decode(codes)
    n = len(pos)
    assert np.all(np.diff(v[:n]) >= 0)                      # positive half, increasing x
    assert np.array_equal(v[n:], -v[:n])                    # sign symmetry
    assert np.abs(v).max() == 448.0
    ratio = x[:n] / float(s[0])
    assert np.all(v[:n][ratio >= 432] == 448.0) and np.all(v[:n][ratio < 431] < 448.0)


def test_fp8_calibration_amax_brute_force():
    vals = [[1.0, -3.0, 0.5], [2.5, -0.25], [-3.25, 0.0]]
    batches = []
    for row in vals:
        x = np.zeros((2, 32), np.float64)
        x[1, : len(row)] = row
        batches.append(_bits_from_f64(x))
    want = max(abs(v) for row in vals for v in row)
    assert oracle.fp8_calibration_amax(batches) == np.float32(want) == np.float32(3.25)
    assert oracle.fp8_calibration_amax(batches[:2]) == np.float32(3.0)
    assert oracle.fp8_calibration_amax([]) == 0.0
    assert oracle.fp8_calibration_amax([np.zeros((3, 64), np.uint16)]) == 0.0
    # the order of the batches does not matter, and -0 counts as 0
    assert oracle.fp8_calibration_amax(batches[::-1]) == np.float32(3.25)
    neg0 = np.full((1, 32), 0x8000, np.uint16)
    assert oracle.fp8_calibration_amax([neg0]) == 0.0
