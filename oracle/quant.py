"""MXFP4 and FP8 per-token quantizers (oracle side).

MXFP4 (the Quark Wan2.2 page, "Quantization formats": OCP MXFP4 weights in
both W4A4 and W4A8, dynamic MXFP4 activations in W4A4; "Results" table rows
marked RTN for the weights). Rows of a [R, K] bf16 matrix are cut into blocks
of 32 consecutive elements along K. For a block with largest magnitude amax:

    E = floor(log2 amax) - 2        (2 = exponent of E2M1's largest value, 6)
    E is clamped to [-127, 127]; an all-zero block takes E = -127
    scale byte = E + 127            (E8M0)
    code_i = E2M1 round-to-nearest-even of v_i / 2^E, saturating at +-6

Packing: element 2t of a block row goes to the low nibble of byte t, element
2t+1 to the high nibble; codes are [R, K/2] bytes, scales [R, K/32] bytes.

FP8 per-token (W4A8 activations; the page names FP8 E4M3 activations, the
per-token scale amax/448 is the reading recorded in the design notes). For row
m with largest magnitude amax_m:

    s_m  = fp32(amax_m) / fp32(448)          IEEE fp32 division
    code = E4M3FN RNE of fp32(x / s_m), saturating at 448 (two roundings:
           the fp32 quotient first, then E4M3FN)
    an all-zero row has s_m = 0 and every code is a signed zero.

FP8 static (the same page's format table names the W4A8 activations FP8 E4M3
"static"; its experimental setup runs a calibration set through the model).
One scale per activation tensor, fixed before inference from the largest
magnitude seen on calibration data:

    amax = max |x| over every calibration batch of the tensor (fp32)
    s    = fp32(amax) / fp32(448)
    code = E4M3FN RNE of fp32(x / s), saturating at +-448: unlike the
           per-token scale, a static one can be exceeded at run time
    s = 0 (all-zero calibration data) gives signed-zero codes, as a zero row
    does per token.
"""

import numpy as np

from .formats import (
    bf16_bits_to_f32,
    bf16_bits_to_f64,
    e2m1_decode,
    e2m1_encode,
    e4m3fn_decode,
    e4m3fn_encode,
    e8m0_decode,
)

BLOCK = 32


def _check_rows(x_bits):
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    if x_bits.ndim != 2:
        raise ValueError("expected a 2-D [rows, K] bf16 bit array")
    if x_bits.shape[1] % BLOCK != 0:
        raise ValueError("K must be a multiple of 32")
    return x_bits


def mxfp4_scale_exponent(amax):
    """Shared exponent E of MX blocks with float64 largest magnitudes ``amax``."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)
    floor_log2 = ex.astype(np.int64) - 1
    e = np.clip(floor_log2 - 2, -127, 127)
    return np.where(amax == 0, -127, e).astype(np.int64)


def mxfp4_quantize(x_bits):
    """bf16 [R, K] (uint16 bits) -> (codes uint8 [R, K/2], scales uint8 [R, K/32])."""
    x_bits = _check_rows(x_bits)
    rows, k = x_bits.shape
    v = bf16_bits_to_f64(x_bits).reshape(rows, k // BLOCK, BLOCK)
    amax = np.abs(v).max(axis=2) if k else np.zeros((rows, 0))
    e = mxfp4_scale_exponent(amax)
    r = v / np.ldexp(1.0, e)[..., None]  # exact: division by a power of two
    codes = e2m1_encode(r).reshape(rows, k)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    scales = (e + 127).astype(np.uint8)
    return packed, scales


def unpack_nibbles(packed):
    """uint8 [R, K/2] -> 4-bit codes uint8 [R, K] (low nibble = even element)."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = packed & 0x0F
    out[:, 1::2] = packed >> 4
    return out


def mxfp4_dequantize(packed, scales):
    """MXFP4 codes + E8M0 scales -> float64 [R, K] values."""
    codes = unpack_nibbles(packed)
    rows, k = codes.shape
    vals = e2m1_decode(codes).reshape(rows, k // BLOCK, BLOCK)
    vals = vals * e8m0_decode(scales)[..., None]
    return vals.reshape(rows, k)


def fp8_per_token_scale(x32):
    """float32 [M, K] -> float32 [M] scales s_m = fp32(amax_m) / fp32(448)."""
    x32 = np.asarray(x32, dtype=np.float32)
    amax = np.abs(x32).max(axis=1) if x32.shape[1] else np.zeros(x32.shape[0], np.float32)
    return (amax.astype(np.float32) / np.float32(448.0)).astype(np.float32)


def fp8_scaled_quotient(x32, s):
    """IEEE fp32 quotients x / s_m (signed zeros for rows whose scale is 0)."""
    x32 = np.asarray(x32, dtype=np.float32)
    s = np.asarray(s, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        r = (x32 / s[:, None]).astype(np.float32)
    zero_row = (s == 0)[:, None]
    return np.where(zero_row, np.copysign(np.float32(0.0), x32), r).astype(np.float32)


def fp8_quantize_per_token(x_bits):
    """bf16 [M, K] (uint16 bits) -> (codes uint8 [M, K] E4M3FN, scales float32 [M])."""
    x_bits = _check_rows(x_bits)
    x32 = bf16_bits_to_f32(x_bits)
    s = fp8_per_token_scale(x32)
    r = fp8_scaled_quotient(x32, s)
    codes = e4m3fn_encode(r.astype(np.float64))
    return codes, s


def fp8_dequantize_per_token(codes, scales):
    """E4M3FN codes [M, K] + float32 scales [M] -> float64 [M, K]."""
    vals = e4m3fn_decode(codes)
    return vals * np.asarray(scales, dtype=np.float32).astype(np.float64)[:, None]


def fp8_calibration_amax(batches):
    """Largest magnitude over calibration batches of bf16 [M, K] (uint16 bits), as float32.

    Every bf16 magnitude is exact in float32, so the result is one of the inputs'
    magnitudes (0 when there is none)."""
    amax = np.float32(0.0)
    for b in batches:
        x32 = bf16_bits_to_f32(_check_rows(b))
        if x32.size:
            amax = max(amax, np.float32(np.abs(x32).max()))
    return np.float32(amax)


def fp8_static_scale(amax):
    """Static per-tensor scale s = fp32(amax) / fp32(448)."""
    return np.float32(np.float32(amax) / np.float32(448.0))


def fp8_quantize_static(x_bits, amax):
    """bf16 [M, K] (uint16 bits) and a calibrated amax -> (codes uint8 [M, K], scales float32 [M]).

    Every row takes the same scale s = amax / 448, so the scale vector is s
    repeated; quotients beyond 448 (and infinite ones, from a tiny s) saturate
    in the E4M3FN encoder."""
    x_bits = _check_rows(x_bits)
    x32 = bf16_bits_to_f32(x_bits)
    s = np.full(x32.shape[0], fp8_static_scale(amax), np.float32)
    r = fp8_scaled_quotient(x32, s)
    codes = e4m3fn_encode(r.astype(np.float64))
    return codes, s
