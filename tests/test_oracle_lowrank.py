"""Pins of the oracle's SVDQuant low-rank branch (CPU only)."""

import numpy as np

import oracle
import synth


def _bits(a):
    return synth.f32_to_bf16_bits(np.asarray(a, np.float32))


def test_down_selects_columns_with_unit_rank_vectors():
    """L1 columns that are unit vectors e_k pick x[:, k] exactly."""
    g = np.random.default_rng(1)
    x = _bits(g.standard_normal((20, 128)))
    picks = [0, 5, 127, 64]
    l1t = np.zeros((32, 128), np.float32)
    for j, k in enumerate(picks):
        l1t[j, k] = 1.0
    t = oracle.lowrank_down(x, _bits(l1t))
    assert t.shape == (20, 32)
    for j, k in enumerate(picks):
        assert np.array_equal(t[:, j], x[:, k])
    assert np.all(t[:, len(picks):] == 0)


def test_up_adds_the_rank_product_and_applies_gelu_to_the_sum():
    y_pre = _bits(np.full((3, 4), 2.0))
    t = _bits([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    l2 = _bits([[1.0, 0.0], [0.0, 3.0], [2.0, 2.0], [0.5, -0.5]])  # [N, r]
    y = oracle.bf16_bits_to_f64(oracle.lowrank_up(y_pre, t, l2))
    want = 2.0 + np.array([[1, 0, 2, 0.5], [0, 3, 2, -0.5], [1, 3, 4, 0]])
    assert np.array_equal(y, want)
    # GELU of 10 rounds to 10 in bf16; GELU of 0 is 0; GELU applies after the sum
    z = oracle.lowrank_up(_bits([[8.0, -2.0]]), _bits([[1.0]]), _bits([[2.0], [2.0]]), oracle.EPI_GELU_TANH)
    assert z[0, 0] == 0x4120 and z[0, 1] == 0x0000


def test_factor_change_of_basis_leaves_the_branch_unchanged():
    """(L1 A, A^-1 L2) with A a permutation times powers of two: T changes exactly by A, the
    product and the layer output do not (a transposed operand would break this)."""
    g = np.random.default_rng(2)
    x = _bits(g.standard_normal((16, 256)))
    l1t = _bits(g.standard_normal((32, 256)) * 0.05)
    l2 = _bits(g.standard_normal((96, 32)) * 0.05)
    y_pre = _bits(g.standard_normal((16, 96)))
    perm = g.permutation(32)
    p2 = np.ldexp(1.0, g.integers(-3, 4, 32))
    l1t_a = _bits(oracle.bf16_bits_to_f64(l1t)[perm] * p2[:, None])          # rows of L1^T: columns of L1 A
    l2_a = _bits(oracle.bf16_bits_to_f64(l2)[:, perm] / p2[None, :])          # columns of L2: rows of A^-1 L2
    t = oracle.lowrank_down(x, l1t)
    t_a = oracle.lowrank_down(x, l1t_a)
    assert np.array_equal(oracle.bf16_bits_to_f64(t_a), oracle.bf16_bits_to_f64(t)[:, perm] * p2[None, :])
    assert np.array_equal(oracle.lowrank_up(y_pre, t, l2), oracle.lowrank_up(y_pre, t_a, l2_a))


def test_exact_dense_weight_through_the_branch():
    """A zero residual and an exactly representable factorization W = L2 L1^T: the layer is the
    bf16 linear x W^T (small integers keep every step exact)."""
    g = np.random.default_rng(3)
    x = _bits(g.integers(-3, 4, (8, 64)))
    l1t = np.zeros((32, 64), np.float32)  # two +-1 entries per rank vector: |T| <= 6
    for j in range(32):
        l1t[j, g.choice(64, 2, replace=False)] = g.choice([-1.0, 1.0], 2)
    l1t = _bits(l1t)
    l2 = _bits(g.integers(-1, 2, (48, 32)))  # |y| <= 192: every value exact in bf16
    w = oracle.bf16_bits_to_f64(l2) @ oracle.bf16_bits_to_f64(l1t)           # [N, K]
    zero_codes = np.zeros((48, 32), np.uint8)
    zero_scales = np.zeros((48, 2), np.uint8)
    a_codes, a_scales = oracle.mxfp4_quantize(x)
    y, y_pre, t = oracle.svdquant_linear(oracle.W4A4, a_codes, a_scales, zero_codes, zero_scales, x, l1t, l2)
    assert np.all(oracle.bf16_bits_to_f64(y_pre) == 0)
    assert np.array_equal(oracle.bf16_bits_to_f64(y), oracle.bf16_bits_to_f64(x) @ w.T)


def test_zero_branch_is_the_plain_layer_rounded_once_more():
    g = np.random.default_rng(4)
    x = synth.activation_bf16(5, 32, 256, ("student_t",))
    w = synth.weight_bf16(5, 64, 256)
    wc, ws = oracle.mxfp4_quantize(w)
    ac, asc = oracle.mxfp4_quantize(x)
    y, y_pre, _ = oracle.svdquant_linear(oracle.W4A4, ac, asc, wc, ws, x, np.zeros((32, 256), np.uint16),
                                         np.zeros((64, 32), np.uint16))
    assert np.array_equal(y, y_pre)
    assert np.array_equal(y_pre, oracle.f64_to_bf16_bits(oracle.qdq_matmul(oracle.W4A4, ac, asc, wc, ws)))


def test_fused_exact_dense_weight():
    """Fused reading: W = L2 L1^T + R with R on the MXFP4 grid and x exact in MXFP4, small
    integers throughout. The layer equals the dense product x W^T plus the bias exactly, whatever
    the rounding of intermediate results."""
    g = np.random.default_rng(6)
    m, n, k, r = 8, 48, 64, 32
    x = _bits(g.choice([-2.0, -1.0, 0.0, 1.0, 2.0, 0.5], (m, k)))
    l1t = np.zeros((r, k), np.float32)
    for j in range(r):
        l1t[j, g.choice(k, 2, replace=False)] = g.choice([-1.0, 1.0], 2)
    l1t = _bits(l1t)
    l2 = _bits(g.integers(-1, 2, (n, r)))
    res = _bits(g.choice([-1.0, 0.0, 0.5, 1.5, 3.0], (n, k)))  # E2M1 values with scale 1 per block
    bias = g.integers(-4, 5, n).astype(np.float64)
    rc, rs = oracle.mxfp4_quantize(res)
    ac, asc = oracle.mxfp4_quantize(x)
    assert np.array_equal(oracle.mxfp4_dequantize(rc, rs), oracle.bf16_bits_to_f64(res))
    assert np.array_equal(oracle.mxfp4_dequantize(ac, asc), oracle.bf16_bits_to_f64(x))
    t = oracle.lowrank_down(x, l1t)
    y = oracle.svdquant_linear_fused(oracle.W4A4, ac, asc, rc, rs, t, l2, bias)
    xf = oracle.bf16_bits_to_f64(x)
    w = oracle.bf16_bits_to_f64(l2) @ oracle.bf16_bits_to_f64(l1t) + oracle.bf16_bits_to_f64(res)
    want = np.zeros((m, n))
    for i in range(m):                       # brute force, element by element
        for c in range(n):
            want[i, c] = sum(xf[i, q] * w[c, q] for q in range(k)) + bias[c]
    assert np.array_equal(y, want)


def test_fused_without_branch_is_the_qdq_product():
    g = np.random.default_rng(7)
    x = synth.activation_bf16(9, 24, 256, ("student_t",))
    w = synth.weight_bf16(9, 64, 256)
    wc, ws = oracle.mxfp4_quantize(w)
    ac, asc = oracle.mxfp4_quantize(x)
    b = g.standard_normal(64)
    for epi in (oracle.EPI_NONE, oracle.EPI_GELU_TANH):
        y = oracle.svdquant_linear_fused(oracle.W4A4, ac, asc, wc, ws, np.zeros((24, 32), np.uint16),
                                         np.zeros((64, 32), np.uint16), b, epi)
        assert np.array_equal(y, oracle.qdq_matmul(oracle.W4A4, ac, asc, wc, ws, b, epi))


def test_fused_and_two_step_readings_agree_when_y_pre_is_exact_in_bf16():
    """With the quantized product exact in bf16 the y_pre rounding of the two-step reading does
    nothing, so the two readings give the same bf16 output; with GELU both apply it to the whole
    sum."""
    g = np.random.default_rng(8)
    m, n, k, r = 16, 64, 128, 64
    x = _bits(g.choice([-1.0, 0.0, 1.0, 2.0], (m, k)))
    res = _bits(g.choice([-0.5, 0.0, 0.5, 1.0], (n, k)))
    rc, rs = oracle.mxfp4_quantize(res)
    ac, asc = oracle.mxfp4_quantize(x)
    l1t = _bits(g.standard_normal((r, k)) * 0.05)
    l2 = _bits(g.standard_normal((n, r)) * 0.05)
    for epi in (oracle.EPI_NONE, oracle.EPI_GELU_TANH):
        y2, y_pre, t = oracle.svdquant_linear(oracle.W4A4, ac, asc, rc, rs, x, l1t, l2, None, epi)
        assert np.array_equal(oracle.bf16_bits_to_f64(y_pre), oracle.qdq_matmul(oracle.W4A4, ac, asc, rc, rs))
        yf = oracle.f64_to_bf16_bits(oracle.svdquant_linear_fused(oracle.W4A4, ac, asc, rc, rs, t, l2, None, epi))
        assert np.array_equal(yf, y2)
