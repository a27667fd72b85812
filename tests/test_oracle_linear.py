"""Pins of the oracle's QDQ matmul, GELU, policy and tolerance (CPU only)."""

from fractions import Fraction

import numpy as np
import torch

import oracle
import synth
from conftest import golden_lines


def _rand_mx_operand(g, rows, k):
    codes = g.integers(0, 256, (rows, k // 2), dtype=np.uint8)
    scales = g.integers(110, 140, (rows, k // 32), dtype=np.uint8)
    return codes, scales


def _exact_mx_value(codes, scales, i, kk):
    byte = int(codes[i, kk // 2])
    nib = byte & 0xF if kk % 2 == 0 else byte >> 4
    mag = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)][nib & 7]
    val = -mag if nib & 8 else mag
    return val * Fraction(2) ** (int(scales[i, kk // 32]) - 127)


def _exact_fp8_value(code):
    code = int(code)
    e, m = (code >> 3) & 15, code & 7
    mag = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -mag if code & 0x80 else mag


def test_qdq_matmul_w4a4_exact_rationals_nonsquare():
    g = np.random.default_rng(0)
    m, n, k = 3, 5, 96
    a, sa = _rand_mx_operand(g, m, k)
    w, sw = _rand_mx_operand(g, n, k)
    bias = np.array([0.5, -1.0, 0.0, 2.0, 0.25])
    y = oracle.qdq_matmul(oracle.W4A4, a, sa, w, sw, bias)
    assert y.shape == (m, n)
    for i in range(m):
        for j in range(n):
            want = sum(_exact_mx_value(a, sa, i, kk) * _exact_mx_value(w, sw, j, kk) for kk in range(k))
            want += Fraction(bias[j])
            assert abs(Fraction(y[i, j]) - want) <= abs(want) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)


def test_qdq_matmul_w4a8_exact_rationals_nonsquare():
    g = np.random.default_rng(1)
    m, n, k = 4, 3, 64
    a = g.integers(0, 256, (m, k), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x12  # no NaN codes
    s = np.array([0.5, 0.013671875, 3.0, 1e-3], np.float32)
    w, sw = _rand_mx_operand(g, n, k)
    y = oracle.qdq_matmul(oracle.W4A8, a, s, w, sw)
    for i in range(m):
        for j in range(n):
            want = sum(_exact_fp8_value(a[i, kk]) * Fraction(float(s[i])) * _exact_mx_value(w, sw, j, kk)
                       for kk in range(k))
            assert abs(Fraction(y[i, j]) - want) <= abs(want) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)


def test_identity_weight_gives_dequantized_activations():
    """W = I is exact in MXFP4 (one 1.0 per row: E = -2, code 4 * 0.25 = 1), so Y = DQ(Q(X))."""
    k = 64
    eye = synth.f32_to_bf16_bits(np.eye(k, dtype=np.float32))
    wq, ws = oracle.mxfp4_quantize(eye)
    assert np.array_equal(oracle.mxfp4_dequantize(wq, ws), np.eye(k))
    g = np.random.default_rng(2)
    x = synth.f32_to_bf16_bits(g.standard_normal((7, k)).astype(np.float32))
    for mode in (oracle.W4A4, oracle.W4A8):
        y, ac, asc = oracle.qlinear(mode, x, wq, ws)
        assert np.array_equal(y, oracle.dequantize_act(mode, ac, asc))


def test_all_ones_closed_form():
    """Every element coded 1.0: y = sum over blocks of 32 * 2^(Ea_j + Ew_j)."""
    k = 128
    a = np.full((2, k // 2), 0x22, np.uint8)
    w = np.full((3, k // 2), 0x22, np.uint8)
    sa = np.array([[127, 128, 120, 130], [100, 127, 127, 127]], np.uint8)
    sw = np.array([[127, 127, 127, 127], [126, 129, 127, 131], [127, 110, 127, 127]], np.uint8)
    y = oracle.qdq_matmul(oracle.W4A4, a, sa, w, sw)
    ea, ew = sa.astype(int) - 127, sw.astype(int) - 127
    for i in range(2):
        for j in range(3):
            assert y[i, j] == sum(32 * 2.0 ** (ea[i, b] + ew[j, b]) for b in range(4))


def test_gelu_tanh_matches_torch():
    y = np.linspace(-12, 12, 4001)
    want = torch.nn.functional.gelu(torch.from_numpy(y), approximate="tanh").numpy()
    assert np.allclose(oracle.gelu_tanh(y), want, rtol=1e-15, atol=1e-15)


def test_qlinear_epilogue_is_gelu_of_matmul():
    g = np.random.default_rng(9)
    x = synth.f32_to_bf16_bits(g.standard_normal((6, 64)).astype(np.float32))
    w = synth.f32_to_bf16_bits(g.standard_normal((10, 64)).astype(np.float32) * 0.02)
    wq, ws = oracle.mxfp4_quantize(w)
    y0, _, _ = oracle.qlinear(oracle.W4A4, x, wq, ws)
    y1, _, _ = oracle.qlinear(oracle.W4A4, x, wq, ws, epilogue=oracle.EPI_GELU_TANH)
    assert np.allclose(y1, torch.nn.functional.gelu(torch.from_numpy(y0), approximate="tanh").numpy(), rtol=1e-14)


def test_policy_table_from_page_counts():
    rows = list(golden_lines("high_tier_policy.txt"))
    names = ["transformer", "transformer_2"]
    table = np.zeros((2, 40), np.uint8)
    for r in rows:
        if r[0] == "w4a8":
            table[names.index(r[1]), [int(b) for b in r[2:]]] = oracle.W4A8
    for r in rows:
        if r[0] == "count":
            e = names.index(r[1])
            n8 = sum(oracle.policy_mode(table, e, b) == oracle.W4A8 for b in range(40))
            assert n8 == int(r[2]) and 40 - n8 == int(r[3])
            assert abs(100.0 * n8 / 40 - float(r[4])) < 1e-9
        if r[0] == "total":
            assert int((table == oracle.W4A8).sum()) == int(r[1]) and table.size == int(r[2])


def test_policy_rejects_other_modes_and_indices():
    table = np.array([[0, 1, 2, 3, 4]], np.uint8)
    assert oracle.policy_mode(table, 0, 0) == oracle.W4A4
    assert oracle.policy_mode(table, 0, 1) == oracle.W4A8
    assert oracle.policy_mode(table, 0, 3) == oracle.TRANSFORM_ON
    for b in (2, 4):
        try:
            oracle.policy_mode(table, 0, b)
            raise AssertionError("accepted a non-linear mode")
        except ValueError:
            pass
    try:
        oracle.policy_mode(table, 1, 0)
        raise AssertionError("accepted an out-of-range expert")
    except IndexError:
        pass


def test_tolerance_check_bounds():
    ref = np.array([1.0, -2.0, 100.0, 0.0])
    rms = np.sqrt(np.mean(ref ** 2))
    ok = ref + 2.0 ** -7 * np.abs(ref) + 0.999e-3 * rms
    assert oracle.output_tolerance_ok(ok, ref)
    bad = ref.copy()
    bad[3] = 1.01e-3 * rms
    assert not oracle.output_tolerance_ok(bad, ref)
    assert not oracle.output_tolerance_ok(np.array([np.nan, 0, 0, 0]), ref)


def test_w4a8_closer_to_bf16_than_w4a4_on_outlier_inputs():
    """Directional sanity (not a parity pin): FP8 activations lose less than MXFP4 ones."""
    x = synth.activation_bf16(99, 128, 512, ("student_t",))
    w = synth.weight_bf16(99, 256, 512)
    wq, ws = oracle.mxfp4_quantize(w)
    ref = oracle.bf16_bits_to_f64(x) @ oracle.bf16_bits_to_f64(w).T

    def sqnr(y):
        return 10 * np.log10(np.sum(ref ** 2) / np.sum((y - ref) ** 2))

    y4, _, _ = oracle.qlinear(oracle.W4A4, x, wq, ws)
    y8, _, _ = oracle.qlinear(oracle.W4A8, x, wq, ws)
    assert sqnr(y8) > sqnr(y4)
