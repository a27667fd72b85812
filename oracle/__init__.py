"""CPU oracle for the MX quantized linear (test infrastructure only).

This package is the slow, plain reference that the GPU library is checked
against. Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import it; the product path (the HIP library and its Python
binding) never does, and the two share no code.

What it computes, following the page "Quark Mixed-Precision Quantization for
Wan2.2 Video Generation on AMD Instinct GPUs" (section "Quantization formats":
W4A4 = OCP MXFP4 weights with dynamic MXFP4 activations, W4A8 = OCP MXFP4
weights with FP8 E4M3 activations; its W4A8 rows were produced by
quantize-dequantize emulation):

* ``formats``  - bf16 bit handling (decode, and the layer's bf16 output
                 rounding), the E2M1 / E4M3FN / E8M0 code tables and a
                 generic round-to-nearest-even into a small binary float format.
* ``quant``    - MXFP4 block quantizer (one E8M0 scale per 32 elements along K)
                 and FP8 E4M3FN quantizers: per-token (scale = row amax / 448)
                 and static (one calibrated scale per tensor, saturating).
* ``transform`` - the transform_on mode: block-diagonal 128-point Hadamard
                 rotation (fp32 butterflies) and SmoothQuant factors ahead of MXFP4.
* ``lowrank``  - SVDQuant's 16-bit low-rank branch beside the quantized
                 product: T = bf16(x L1), y = bf16(epilogue(y_pre + T L2)),
                 or with T L2 inside the product's sums (one rounding).
* ``select``   - calibration-driven block selection: block-replay SQNR (OFF
                 = plain MXFP4, ON = transform) and the tiered rule ladder that
                 emits the policy artifact.
* ``linear``   - dequantize-then-fp64 matmul (the QDQ result), tanh-GELU, the
                 per-block policy lookup and the output tolerance check.

Every floating-point step is float64 unless the format fixes fp32 (the FP8
per-token scale and quotient). Parity of every function is pinned by the
``-m "not gpu"`` tests against closed forms, brute force and library routines.
"""

from .formats import (
    E2M1_MAGNITUDES,
    bf16_bits_to_f64,
    bf16_bits_to_f32,
    e2m1_decode,
    e4m3fn_decode,
    e8m0_decode,
    round_to_binary_format,
    e2m1_encode,
    e4m3fn_encode,
    f64_to_bf16_bits,
    BF16_MAX,
)
from .quant import (
    mxfp4_quantize,
    mxfp4_dequantize,
    mxfp4_scale_exponent,
    fp8_quantize_per_token,
    fp8_dequantize_per_token,
    fp8_per_token_scale,
    fp8_scaled_quotient,
    fp8_calibration_amax,
    fp8_static_scale,
    fp8_quantize_static,
    unpack_nibbles,
)
from .transform import (
    fwht128_f32,
    hadamard_channel_amax,
    smoothquant_factors,
    hadamard_transform_bf16,
    mxfp4_quantize_hadamard,
    INV_SQRT_BLOCK,
)
from .lowrank import (
    lowrank_down,
    lowrank_up,
    svdquant_linear,
    svdquant_linear_fused,
)
from .select import (
    TIERS,
    BF16_MODE,
    sqnr_sums,
    sqnr_db,
    select_mode,
    select_policy,
    block_replay_sums,
)
from .linear import (
    W4A4,
    W4A8,
    TRANSFORM_ON,
    EPI_NONE,
    EPI_GELU_TANH,
    gelu_tanh,
    qdq_matmul,
    quantize_act,
    dequantize_act,
    qlinear,
    qlinear_transform,
    policy_mode,
    output_tolerance_ok,
    output_error_report,
)

__all__ = [name for name in dir() if not name.startswith("_")]
