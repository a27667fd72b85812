"""The ``transform_on`` mode: fixed Hadamard rotation, then SmoothQuant, before MXFP4 (oracle side).

The Quark Wan2.2 page ("Calibration-driven block selection", "Mixed-Precision
selection", "Practical workflow" step 6) keeps a block on W4A4 but turns a
transform on when it lifts the block's SQNR: a fixed (not learned) Hadamard
rotation, R1 on the residual stream and R2 inside the 128-wide attention head
dimension, followed by SmoothQuant, which moves per-channel activation outliers
into the weights. For one linear y = x W^T this is an orthogonal change of
basis of the K dimension plus a per-channel rescale, applied to the activation
online and to the weight offline, so that the product is unchanged:

    x_t = (x H) / lambda,     W_t = (W H) * lambda,     x_t W_t^T = x W^T

Readings recorded in the design notes:

* H is block diagonal: one normalized 128-point Walsh-Hadamard matrix per 128
  consecutive elements of K (R2's head dimension is 128; R1's dimension, 5120,
  is no power of two, and 128 is one MXFP4 code panel).
* lambda_k = sqrt(amax_x_k / amax_w_k): SmoothQuant with migration strength
  0.5, from the per-channel maxima of the rotated calibration activations and
  of the rotated weight; lambda_k = 1 where either maximum is 0.
* The arithmetic is fp32 in a fixed order, so that both sides take the same
  rounding decisions before the codes: the unnormalized transform is computed
  by butterflies (stage h = 1, 2, 4, ..., 64: a + b and a - b of the elements
  h apart, each an IEEE fp32 operation), each channel is then multiplied by one
  fp32 factor (act_mult_k = RN(RN(1 / lambda_k) * RN(1 / sqrt(128))) for the
  activation, w_mult_k = RN(lambda_k * RN(1 / sqrt(128))) for the weight), and
  the result is rounded to bf16, the activation dtype, before the usual MXFP4
  quantizer.
* An output of the rotation that cancels exactly is +0: the factor is applied
  as RN(t * mult + 0), which leaves every nonzero product (and the sign of one
  that underflows) as RN(t * mult) and turns an exact zero into +0. The sign of
  an exactly cancelling sum says nothing about the data, and the IEEE rules
  would tie it to the order of the butterflies.
"""

import numpy as np

from .formats import bf16_bits_to_f32, f64_to_bf16_bits
from .quant import mxfp4_quantize

BLOCK = 128
INV_SQRT_BLOCK = np.float32(1.0 / np.sqrt(128.0))  # RN(1 / sqrt(128)) in fp32


def _check_k(x):
    x = np.asarray(x)
    if x.ndim != 2 or x.shape[1] % BLOCK != 0:
        raise ValueError("expected [rows, K] with K a multiple of 128")
    return x


def fwht128_f32(x32):
    """Unnormalized Walsh-Hadamard transform of each 128-element block along K, in fp32 butterflies.

    out[., 128 b + k] = sum_j (-1)^popcount(j & k) x[., 128 b + j], computed stage by
    stage (h = 1, 2, 4, ..., 64), every add and subtract rounded to fp32."""
    v = _check_k(np.asarray(x32, dtype=np.float32)).copy()
    rows, k = v.shape
    v = v.reshape(rows, k // BLOCK, BLOCK)
    h = 1
    while h < BLOCK:
        w = v.reshape(rows, k // BLOCK, BLOCK // (2 * h), 2, h)
        a = w[:, :, :, 0, :].copy()
        b = w[:, :, :, 1, :].copy()
        w[:, :, :, 0, :] = a + b  # float32 + float32 -> float32 (IEEE, round to nearest)
        w[:, :, :, 1, :] = a - b
        h *= 2
    return v.reshape(rows, k)


def hadamard_channel_amax(batches):
    """Per-channel max |fwht128(x)| over calibration batches of bf16 [M, K] -> float32 [K]."""
    amax = None
    for b in batches:
        t = np.abs(fwht128_f32(bf16_bits_to_f32(_check_k(b))))
        m = t.max(axis=0) if t.shape[0] else np.zeros(t.shape[1], np.float32)
        amax = m if amax is None else np.maximum(amax, m)
    return amax


def smoothquant_factors(act_amax, w_amax):
    """(act_mult, w_mult) float32 [K] from the rotated per-channel maxima (migration strength 0.5)."""
    ax = np.asarray(act_amax, dtype=np.float32)
    aw = np.asarray(w_amax, dtype=np.float32)
    ok = (ax > 0) & (aw > 0)
    with np.errstate(divide="ignore", invalid="ignore"):
        lam = np.where(ok, np.sqrt(np.where(ok, ax, 1) / np.where(ok, aw, 1)), np.float32(1)).astype(np.float32)
    inv = (np.float32(1) / lam).astype(np.float32)
    act_mult = (inv * INV_SQRT_BLOCK).astype(np.float32)
    w_mult = (lam * INV_SQRT_BLOCK).astype(np.float32)
    return act_mult, w_mult


def hadamard_transform_bf16(x_bits, mult):
    """bf16 [R, K] -> the transformed tensor in bf16: RN_bf16(RN_fp32(fwht128_f32(x) * mult + 0)) (uint16 bits).

    The fp32 product is exact in float64, so adding +0 there and rounding once
    to fp32 is RN(t * mult + 0): an exact zero becomes +0, anything else is the
    fp32 product."""
    t = fwht128_f32(bf16_bits_to_f32(_check_k(x_bits))).astype(np.float64)
    t = (t * np.asarray(mult, dtype=np.float32).astype(np.float64)[None, :] + 0.0).astype(np.float32)
    return f64_to_bf16_bits(t.astype(np.float64))


def mxfp4_quantize_hadamard(x_bits, mult):
    """Transform (rotation + per-channel factor), bf16 rounding, then the MXFP4 quantizer.

    With act_mult this is the transform_on activation quantizer; with w_mult it
    packs the weight of a transform_on linear."""
    return mxfp4_quantize(hadamard_transform_bf16(x_bits, mult))
