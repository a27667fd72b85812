"""Exhaustive GPU checks of the conversion instructions the quantizers use.

The MXFP4 quantizer rounds with gfx950's scaled bf16 -> FP4 conversion, the
FP8 quantizer with its fp32 -> E4M3 conversion, and the transformed MXFP4
quantizer (and every bf16 output) with its fp32 -> bf16 conversion. Each is compared on the
GPU with the software rounding of mxq_convert.h over its whole input domain
(every finite bf16 at every block scale that can hold it; every fp32 quotient
the FP8 quantizer can produce, both signs). The host build of that software
rounding is itself checked exhaustively against the oracle (test_hostcheck),
so the instructions are tied to the pages' rounding rule on every input.
"""

import ctypes
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hip", "libmxq_convcheck.so")


@pytest.fixture(scope="module")
def lib():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    assert os.path.exists(LIB), f"{LIB} missing: run python -m mx_bit_quantized_amd._build"
    return ctypes.CDLL(LIB)


def _run(lib, name):
    counts = np.zeros(2, np.uint64)
    first = np.zeros(24, np.uint32)
    rc = getattr(lib, name)(counts.ctypes.data_as(ctypes.c_void_p), first.ctypes.data_as(ctypes.c_void_p))
    assert rc == 0, f"{name}: HIP error {rc}"
    return int(counts[0]), int(counts[1]), first.reshape(8, 3)


def test_fp4_scaled_conversion_matches_rounding_rule(lib):
    print("[case] fp4 conversion, every finite bf16 x every scale byte", flush=True)
    bad, cases, first = _run(lib, "mxq_check_fp4")
    # scale byte b admits the magnitudes with exponent field 0 .. b + 2, both signs
    assert cases == sum((b + 3) * 128 * 2 for b in range(253)), cases
    assert bad == 0, f"{bad} mismatches of {cases}; first (case, want, got): {first[:min(bad, 8)].tolist()}"


def test_fp8_conversion_matches_rounding_rule(lib):
    print("[case] fp8 conversion, every fp32 with |q| <= 464", flush=True)
    bad, cases, first = _run(lib, "mxq_check_fp8")
    assert cases == 2 * (0x43E80000 + 1), cases  # every fp32 pattern from +0 to 464.0, and its negative
    assert bad == 0, f"{bad} mismatches of {cases}; first (case, want, got): {first[:min(bad, 8)].tolist()}"


def test_bf16_conversion_matches_rounding_rule(lib):
    print("[case] bf16 conversion, every non-NaN fp32", flush=True)
    bad, cases, first = _run(lib, "mxq_check_bf16")
    assert cases == 2 * (0x7F800000 + 1), cases  # +0 .. +inf and their negatives
    assert bad == 0, f"{bad} mismatches of {cases}; first (case, want, got): {first[:min(bad, 8)].tolist()}"
