"""Pins of the oracle's transform_on mode: 128-point Hadamard rotation in fp32
butterflies, SmoothQuant factors and the transformed MXFP4 quantizer (CPU only)."""

import numpy as np
import pytest
import scipy.linalg

import oracle
import synth
from conftest import golden_lines

H128 = scipy.linalg.hadamard(128).astype(np.float64)  # Sylvester order: (-1)^popcount(j & k)


def _exact_fwht(x64):
    r, k = x64.shape
    return (x64.reshape(r, k // 128, 128) @ H128.T).reshape(r, k)


def test_fwht_equals_hadamard_matrix_on_exact_inputs():
    """Small integers: every butterfly sum is exact in fp32, so the result is H x exactly."""
    g = np.random.default_rng(1)
    x = g.integers(-1000, 1000, (16, 512)).astype(np.float32)
    got = oracle.fwht128_f32(x)
    assert got.dtype == np.float32
    assert np.array_equal(got.astype(np.float64), _exact_fwht(x.astype(np.float64)))


def test_fwht_is_its_own_inverse_up_to_128():
    g = np.random.default_rng(2)
    x = g.integers(-500, 500, (8, 256)).astype(np.float32)
    assert np.array_equal(oracle.fwht128_f32(oracle.fwht128_f32(x)), 128 * x)


def test_fwht_unit_vectors_give_hadamard_rows():
    x = np.eye(128, dtype=np.float32)
    assert np.array_equal(oracle.fwht128_f32(x).astype(np.float64), H128)  # H is symmetric


def test_fwht_golden_rounding_order():
    x = np.zeros((1, 128), np.float32)
    want = {}
    for row in golden_lines("fwht128.txt"):
        if row[0] == "in":
            x[0, int(row[1])] = float(row[2])
        else:
            want[int(row[1])] = float(row[2])
    got = oracle.fwht128_f32(x)[0]
    for k in range(128):
        assert got[k] == np.float32(want[k % 4]), (k, got[k])
    assert not np.array_equal(got.astype(np.float64), _exact_fwht(x.astype(np.float64))[0])


def test_fwht_error_bound_on_random_inputs():
    """|fp32 butterflies - exact| <= 7 u sum|x| per output (7 stages, unit roundoff u = 2^-24)."""
    g = np.random.default_rng(3)
    x = (g.standard_normal((32, 384)) * np.ldexp(1.0, g.integers(-20, 20, (32, 384)))).astype(np.float32)
    got = oracle.fwht128_f32(x).astype(np.float64)
    exact = _exact_fwht(x.astype(np.float64))
    bound = 7 * 2.0 ** -24 * np.abs(x.astype(np.float64)).reshape(32, 3, 128).sum(axis=2)
    err = np.abs(got - exact).reshape(32, 3, 128)
    assert np.all(err <= bound[:, :, None] * 1.0000001)
    assert np.any(err > 0)  # the sample does round


def test_smoothquant_factors_closed_forms():
    c0 = np.float32(1.0 / np.sqrt(128.0))
    ax = np.array([3.0, 8.0, 0.0, 5.0, 1.0, 2.0 ** -10], np.float32)
    aw = np.array([3.0, 2.0, 7.0, 0.0, 4.0, 2.0 ** -20], np.float32)
    am, wm = oracle.smoothquant_factors(ax, aw)
    # lambda = 1, 2, 1 (zero act max), 1 (zero weight max), 0.5, 32
    lam = [1.0, 2.0, 1.0, 1.0, 0.5, 32.0]
    for i, l in enumerate(lam):
        assert am[i] == np.float32(np.float32(1.0 / l) * c0), i
        assert wm[i] == np.float32(np.float32(l) * c0), i
    assert am.dtype == np.float32 and wm.dtype == np.float32


def test_smoothquant_factor_product_and_lambda_rounding():
    """act_mult * w_mult = 1/128 up to a few ulps, and lambda is the correctly rounded sqrt."""
    g = np.random.default_rng(4)
    ax = np.ldexp(g.uniform(1, 2, 2000), g.integers(-30, 30, 2000)).astype(np.float32)
    aw = np.ldexp(g.uniform(1, 2, 2000), g.integers(-30, 30, 2000)).astype(np.float32)
    am, wm = oracle.smoothquant_factors(ax, aw)
    prod = am.astype(np.float64) * wm.astype(np.float64) * 128
    assert np.all(np.abs(prod - 1) < 4 * 2.0 ** -23)
    # lambda recovered from w_mult: within one rounding of sqrt(ax / aw) in float64
    lam = wm.astype(np.float64) / np.float64(np.float32(1 / np.sqrt(128)))
    assert np.all(np.abs(lam / np.sqrt(ax.astype(np.float64) / aw.astype(np.float64)) - 1) < 3 * 2.0 ** -24)


def test_transform_keeps_the_product():
    """Without the bf16 rounding, x_t W_t^T = x W^T (orthogonal rotation, reciprocal rescale)."""
    g = np.random.default_rng(5)
    x = synth.activation_bf16(11, 24, 256, ("student_t",))
    w = synth.weight_bf16(11, 40, 256)
    x32 = oracle.bf16_bits_to_f32(x)
    w32 = oracle.bf16_bits_to_f32(w)
    ax = oracle.hadamard_channel_amax([x])
    aw = oracle.hadamard_channel_amax([w])
    am, wm = oracle.smoothquant_factors(ax, aw)
    xt = oracle.fwht128_f32(x32).astype(np.float64) * am
    wt = oracle.fwht128_f32(w32).astype(np.float64) * wm
    ref = x32.astype(np.float64) @ w32.astype(np.float64).T
    got = xt @ wt.T
    scale = np.abs(x32).astype(np.float64) @ np.abs(w32).astype(np.float64).T
    assert np.all(np.abs(got - ref) <= 1e-5 * scale + 1e-30)


def test_channel_amax_brute_force():
    g = np.random.default_rng(6)
    b1 = synth.f32_to_bf16_bits(g.integers(-50, 50, (5, 256)).astype(np.float32))
    b2 = synth.f32_to_bf16_bits(g.integers(-50, 50, (3, 256)).astype(np.float32))
    got = oracle.hadamard_channel_amax([b1, b2])
    allx = np.concatenate([oracle.bf16_bits_to_f64(b1), oracle.bf16_bits_to_f64(b2)])
    want = np.abs(_exact_fwht(allx)).max(axis=0)
    assert np.array_equal(got.astype(np.float64), want)
    assert np.array_equal(oracle.hadamard_channel_amax([b2, b1]), got)


def test_transformed_bf16_and_codes_on_exact_inputs():
    """Integer inputs and power-of-two factors: the transformed bf16 values are the exact H x times
    the factor, rounded once to bf16, and the codes are the plain quantizer's codes of those values."""
    g = np.random.default_rng(7)
    x = synth.f32_to_bf16_bits(g.integers(-100, 100, (6, 256)).astype(np.float32))
    mult = np.ldexp(1.0, g.integers(-6, 2, 256)).astype(np.float32)
    got = oracle.hadamard_transform_bf16(x, mult)
    want = oracle.f64_to_bf16_bits(_exact_fwht(oracle.bf16_bits_to_f64(x)) * mult)
    assert np.array_equal(got, want)
    c, s = oracle.mxfp4_quantize_hadamard(x, mult)
    c2, s2 = oracle.mxfp4_quantize(want)
    assert np.array_equal(c, c2) and np.array_equal(s, s2)


def test_transform_lifts_sqnr_on_outlier_channels():
    """The page's reason for the transform: on activations with heavy outlier channels the
    rotated + smoothed W4A4 product is closer to the exact one than plain MXFP4."""
    x = synth.activation_bf16(12, 128, 512, ("scaled", 4, 20.0))
    w = synth.weight_bf16(12, 96, 512)
    ref = oracle.bf16_bits_to_f64(x) @ oracle.bf16_bits_to_f64(w).T
    pc, ps = oracle.mxfp4_quantize(x)
    wc, ws = oracle.mxfp4_quantize(w)
    y_plain = oracle.qdq_matmul(oracle.W4A4, pc, ps, wc, ws)
    am, wm = oracle.smoothquant_factors(oracle.hadamard_channel_amax([x]), oracle.hadamard_channel_amax([w]))
    tc, ts = oracle.mxfp4_quantize_hadamard(x, am)
    twc, tws = oracle.mxfp4_quantize_hadamard(w, wm)
    y_t = oracle.qdq_matmul(oracle.W4A4, tc, ts, twc, tws)
    sqnr = lambda y: 10 * np.log10((ref ** 2).sum() / ((y - ref) ** 2).sum())
    assert sqnr(y_t) > sqnr(y_plain) + 1.0, (sqnr(y_t), sqnr(y_plain))


def test_exact_zero_outputs_are_positive_and_underflow_keeps_its_sign():
    """An exactly cancelling rotation output is +0 whatever the IEEE signs of the
    butterflies; a nonzero product that rounds to zero keeps its sign."""
    x = np.zeros((3, 128), np.float32)
    x[0, :] = -0.0                  # every sum of -0's is -0 under IEEE; here it is +0
    x[1, 0], x[1, 1] = 3.0, 3.0     # outputs with (-1)^k in bit 0 cancel exactly
    x[2, 0] = -1.0                  # every output is -1 (times its sign pattern)
    bits = synth.f32_to_bf16_bits(x)
    bits[0, :] = 0x8000
    t_raw = oracle.fwht128_f32(oracle.bf16_bits_to_f32(bits))
    assert np.signbit(t_raw[0, 0])  # the butterflies alone give -0
    tiny = np.full(128, np.float32(2.0 ** -140), np.float32)  # -1 * 2^-140 underflows bf16 to -0
    out = oracle.hadamard_transform_bf16(bits, tiny)
    assert np.all(out[0] == 0x0000)
    assert np.all(out[1, 1::2] == 0x0000)                       # 3 - 3
    # row 2 transforms to -1 everywhere; times 2^-140 it is a nonzero fp32 that
    # rounds to zero in bf16 (below half of 2^-133), keeping its sign
    assert np.all(out[2] == 0x8000)


def test_rejects_k_not_multiple_of_128():
    with pytest.raises(ValueError):
        oracle.fwht128_f32(np.zeros((2, 96), np.float32))
