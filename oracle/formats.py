"""Element and scale formats of the MX quantized linear (oracle side).

Sources. The Quark Wan2.2 page ("Quark Mixed-Precision Quantization for Wan2.2
Video Generation on AMD Instinct GPUs", section "Quantization formats") names
the formats: OCP MXFP4 for weights and W4A4 activations (its reference [7], the
OCP Microscaling Formats v1.0 specification) and FP8 E4M3 for W4A8
activations. The bit layouts below are those of the OCP definitions:

* E2M1 (FP4): sign bit 3, two exponent bits with bias 1, one mantissa bit.
  Exponent field 0 is subnormal (0 or 0.5); the magnitudes are
  0, 0.5, 1, 1.5, 2, 3, 4, 6. No inf or NaN.
* E4M3FN (FP8): sign bit 7, four exponent bits with bias 7, three mantissa
  bits. Exponent field 0 is subnormal (m/8 * 2^-6); 0x7F and 0xFF are NaN;
  the largest finite magnitude is 448 (0x7E).
* E8M0 (shared scale): an unsigned biased exponent, value 2^(u - 127);
  u = 255 is NaN.

bf16 values are carried as their uint16 bit patterns, since NumPy has no bf16.
"""

import numpy as np

# Magnitudes of the eight non-negative E2M1 codes, in code order.
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def bf16_bits_to_f32(bits):
    """uint16 bf16 patterns -> float32 values (exact: bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def bf16_bits_to_f64(bits):
    """uint16 bf16 patterns -> float64 values (exact)."""
    return bf16_bits_to_f32(bits).astype(np.float64)


def e2m1_decode(codes):
    """4-bit E2M1 codes (0..15, in a uint8 array) -> float64 values."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = (c >> 3) & 1
    exp = (c >> 1) & 3
    man = c & 1
    subnormal = 0.5 * man
    normal = (1.0 + 0.5 * man) * np.ldexp(1.0, exp - 1)
    mag = np.where(exp == 0, subnormal, normal)
    return np.where(sign == 1, -mag, mag)


def e4m3fn_decode(codes):
    """8-bit E4M3FN codes -> float64 values (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = (c >> 7) & 1
    exp = (c >> 3) & 15
    man = c & 7
    subnormal = (man / 8.0) * 2.0 ** -6
    normal = (1.0 + man / 8.0) * np.ldexp(1.0, exp - 7)
    mag = np.where(exp == 0, subnormal, normal)
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def e8m0_decode(codes):
    """8-bit E8M0 scale codes -> float64 powers of two (NaN for 255)."""
    u = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    val = np.ldexp(1.0, u - 127)
    return np.where(u == 255, np.nan, val)


def round_to_binary_format(r, mbits, emin, maxval):
    """Round float64 values into a binary float format, ties to even, saturating.

    The format has ``mbits`` explicit mantissa bits, smallest normal exponent
    ``emin`` (the subnormal range shares emin's quantum) and largest finite
    magnitude ``maxval``. Each |r| is rounded to the nearest multiple of the
    quantum of its binade, 2^(max(floor(log2|r|), emin) - mbits), with ties
    going to the even multiple (an even significand, hence an even code);
    results above ``maxval`` are clamped to it. The sign of r is kept, also
    for values that round to zero. float64 holds every operand here exactly.
    """
    r = np.asarray(r, dtype=np.float64)
    a = np.abs(r)
    _, ex = np.frexp(a)  # a = f * 2^ex with f in [0.5, 1): floor(log2 a) = ex - 1
    e = np.maximum(ex.astype(np.int64) - 1, emin)
    quantum = np.ldexp(1.0, e - mbits)
    q = np.rint(a / quantum) * quantum  # np.rint rounds half to even
    q = np.minimum(q, maxval)
    return np.copysign(q, r)


def _encode_from_table(q, table, sign_shift):
    """Signed representable values -> codes via the sorted magnitude table."""
    mag = np.abs(q)
    idx = np.searchsorted(table, mag)
    if not np.array_equal(table[np.minimum(idx, len(table) - 1)], mag):
        raise ValueError("value is not representable in the format")
    sign = np.signbit(q).astype(np.int64)
    return (idx.astype(np.int64) | (sign << sign_shift)).astype(np.uint8)


def e2m1_encode(r):
    """float64 values (already divided by the block scale) -> E2M1 codes (RNE, saturating at 6)."""
    q = round_to_binary_format(r, mbits=1, emin=0, maxval=6.0)
    return _encode_from_table(q, E2M1_MAGNITUDES, 3)


_E4M3_MAGNITUDES = e4m3fn_decode(np.arange(0x7F, dtype=np.uint8))  # codes 0x00..0x7E, increasing


def e4m3fn_encode(r):
    """float64 values -> E4M3FN codes (RNE, saturating at 448, never NaN)."""
    q = round_to_binary_format(r, mbits=3, emin=-6, maxval=448.0)
    return _encode_from_table(q, _E4M3_MAGNITUDES, 7)


BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def f64_to_bf16_bits(r):
    """float64 values -> bf16 bit patterns, IEEE round to nearest even.

    The layer's output is stored in bf16 (8 exponent bits, 7 mantissa bits,
    subnormals from 2^-133). Magnitudes that round above the largest finite
    value become infinities, as in IEEE rounding; NaN stays NaN.
    """
    r = np.asarray(r, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        q = round_to_binary_format(r, mbits=7, emin=-126, maxval=np.inf)
        q = np.where(np.abs(q) > BF16_MAX, np.copysign(np.inf, r), q)
        bits = (q.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return bits
