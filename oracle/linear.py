"""Quantized linear: QDQ matmul, tanh-GELU, policy lookup, tolerance (oracle side).

The Quark Wan2.2 page ("Quantization formats", kernel note) evaluated W4A8 by
quantize-dequantize emulation and runs W4A4 natively; both reach the same
mathematical result, which this module writes out directly:

    y[m, n] = sum_k deqA[m, k] * deqW[n, k]  (+ bias[n])     in float64

with deqW = e2m1(w) * 2^Ew (MXFP4 weights, both modes), deqA = e2m1(a) * 2^Ea
(W4A4) or e4m3(a) * s_m (W4A8). Every product of decoded operands is exact in
float64, so the only rounding is the float64 summation.

The policy table is the per-expert, per-block artifact of the page's "Practical
workflow" (step 6): one mode per (expert, block). Only the W4A4 and W4A8 values
reach the quantized linear; the page's ``bf16`` and ``transform_on`` values are
not modes of this layer.

The FFN's first projection is followed by GELU; the tanh form used here is
0.5 * y * (1 + tanh(sqrt(2/pi) * (y + 0.044715 * y^3))).
"""

import numpy as np

from .quant import (
    fp8_dequantize_per_token,
    fp8_quantize_per_token,
    mxfp4_dequantize,
    mxfp4_quantize,
)

W4A4 = 0
W4A8 = 1
TRANSFORM_ON = 3  # W4A4 behind the Hadamard + SmoothQuant transform (policy value)
EPI_NONE = 0
EPI_GELU_TANH = 1


def gelu_tanh(y):
    """tanh-approximated GELU in float64."""
    y = np.asarray(y, dtype=np.float64)
    c = np.sqrt(2.0 / np.pi)
    return 0.5 * y * (1.0 + np.tanh(c * (y + 0.044715 * y ** 3)))


def quantize_act(mode, x_bits):
    """Activation quantizer of one mode: W4A4 -> MXFP4, W4A8 -> FP8 per-token."""
    if mode == W4A4:
        return mxfp4_quantize(x_bits)
    if mode == W4A8:
        return fp8_quantize_per_token(x_bits)
    raise ValueError(f"mode {mode} is not a quantized-linear mode")


def dequantize_act(mode, codes, scales):
    if mode == W4A4:
        return mxfp4_dequantize(codes, scales)
    if mode == W4A8:
        return fp8_dequantize_per_token(codes, scales)
    raise ValueError(f"mode {mode} is not a quantized-linear mode")


def qdq_matmul(mode, a_codes, a_scales, w_codes, w_scales, bias=None, epilogue=EPI_NONE):
    """float64 y [M, N] from quantized activations and MXFP4 weights."""
    deq_a = dequantize_act(mode, a_codes, a_scales)
    deq_w = mxfp4_dequantize(w_codes, w_scales)
    y = deq_a @ deq_w.T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    if epilogue == EPI_GELU_TANH:
        y = gelu_tanh(y)
    elif epilogue != EPI_NONE:
        raise ValueError(f"unknown epilogue {epilogue}")
    return y


def policy_mode(table, expert, block):
    """Mode of (expert, block) in a [n_experts, n_blocks] table.

    W4A4, W4A8 and transform_on (the artifact's third quantized value) are
    modes of the layer; the artifact's bf16 entry (2) and anything else are
    rejected."""
    table = np.asarray(table)
    if not (0 <= expert < table.shape[0] and 0 <= block < table.shape[1]):
        raise IndexError("policy index out of range")
    mode = int(table[expert, block])
    if mode not in (W4A4, W4A8, TRANSFORM_ON):
        raise ValueError(f"policy mode {mode} is not W4A4, W4A8 or transform_on")
    return mode


def qlinear(mode, x_bits, w_codes, w_scales, bias=None, epilogue=EPI_NONE):
    """Quantize x with the mode's activation format, then the QDQ matmul.

    Returns (y float64, a_codes, a_scales)."""
    a_codes, a_scales = quantize_act(mode, x_bits)
    y = qdq_matmul(mode, a_codes, a_scales, w_codes, w_scales, bias, epilogue)
    return y, a_codes, a_scales


def output_error_report(y, y_ref):
    """Worst ratio of |y - y_ref| to the allowed bound 2^-7 |y_ref| + 1e-3 rms(y_ref)."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(y_ref ** 2))) if y_ref.size else 0.0
    bound = 2.0 ** -7 * np.abs(y_ref) + 1e-3 * rms
    err = np.abs(y - y_ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / bound, np.where(err > 0, np.inf, 0.0))
    worst = float(ratio.max()) if ratio.size else 0.0
    return {
        "finite": bool(np.all(np.isfinite(y))),
        "worst_ratio": worst,
        "max_abs_err": float(err.max()) if err.size else 0.0,
        "rms_ref": rms,
        "n": int(y.size),
    }


def output_tolerance_ok(y, y_ref):
    """True iff y is finite and |y - y_ref| <= 2^-7 |y_ref| + 1e-3 rms(y_ref) everywhere."""
    rep = output_error_report(y, y_ref)
    return rep["finite"] and rep["worst_ratio"] <= 1.0


def qlinear_transform(mode, x_bits, w_codes, w_scales, act_mult=None, bias=None, epilogue=EPI_NONE):
    """qlinear for a policy that may hold transform_on blocks.

    transform_on quantizes x with the transformed MXFP4 quantizer (act_mult) and
    multiplies with the weight packed by it (w_mult); the product is the W4A4
    QDQ matmul of those codes. Other modes are qlinear. Returns (y, a_codes, a_scales)."""
    if mode != TRANSFORM_ON:
        return qlinear(mode, x_bits, w_codes, w_scales, bias, epilogue)
    from .transform import mxfp4_quantize_hadamard

    a_codes, a_scales = mxfp4_quantize_hadamard(x_bits, act_mult)
    y = qdq_matmul(W4A4, a_codes, a_scales, w_codes, w_scales, bias, epilogue)
    return y, a_codes, a_scales
