"""Pins of the oracle's calibration-driven block selection: SQNR, the tiered
rule ladder and the block replay (CPU only)."""

import math

import numpy as np
import pytest

import oracle
import synth
from conftest import golden_lines

NAMES = {"bf16": oracle.BF16_MODE, "w4a8": oracle.W4A8, "w4a4": oracle.W4A4, "transform_on": oracle.TRANSFORM_ON}


def test_tiers_and_rule_cases_from_the_page():
    tiers, cases = {}, []
    for row in golden_lines("select_rules.txt"):
        if row[0] == "tier":
            tiers[row[1]] = tuple(float(v) for v in row[2:5])
        else:
            cases.append((row[1], float(row[2]), float(row[3]), NAMES[row[4]]))
    assert tiers == oracle.TIERS
    assert len(cases) >= 15
    for tier, off, on, want in cases:
        assert oracle.select_mode(off, on, tier) == want, (tier, off, on)


def test_select_policy_table():
    off = np.array([[11.0, 24.0, 30.0], [26.0, 13.0, 40.0]])
    on = np.array([[11.5, 24.5, 31.0], [26.4, 12.0, 40.6]])
    want = np.array([[2, 1, 3], [0, 1, 3]], np.uint8)
    assert np.array_equal(oracle.select_policy(off, on, "high"), want)
    # a lower tier promotes fewer blocks
    assert np.array_equal(oracle.select_policy(off, on, "low"), np.array([[1, 0, 3], [0, 1, 3]], np.uint8))


def test_sqnr_closed_forms():
    ref = np.ones(100)
    s, n = oracle.sqnr_sums(ref + 0.1, ref)
    assert s == 100.0 and abs(n - 1.0) < 1e-12
    assert abs(oracle.sqnr_db(s, n) - 20.0) < 1e-9
    assert oracle.sqnr_db(*oracle.sqnr_sums(ref, ref)) == math.inf
    assert oracle.sqnr_db(*oracle.sqnr_sums(np.ones(4), np.zeros(4))) == -math.inf
    assert oracle.sqnr_db(0.0, 0.0) == math.inf
    # y = 0 has the signal's energy as noise: 0 dB
    assert oracle.sqnr_db(*oracle.sqnr_sums(np.zeros(10), np.arange(10.0))) == 0.0
    # invariant under a common scale
    g = np.random.default_rng(1)
    r = g.standard_normal(500)
    y = r + 0.03 * g.standard_normal(500)
    a = oracle.sqnr_db(*oracle.sqnr_sums(y, r))
    b = oracle.sqnr_db(*oracle.sqnr_sums(7.5 * y, 7.5 * r))
    assert abs(a - b) < 1e-9


def _block(seed, m, dims, outliers):
    """A synthetic block: linears (x, w, y_ref) with y_ref the BF16 product (float64 rounded to bf16)."""
    lins = []
    for i, (n, k) in enumerate(dims):
        x = synth.activation_bf16(seed + i, m, k, outliers)
        w = synth.weight_bf16(seed + i, n, k)
        y_ref = oracle.f64_to_bf16_bits(oracle.bf16_bits_to_f64(x) @ oracle.bf16_bits_to_f64(w).T)
        lins.append((x, w, oracle.bf16_bits_to_f64(y_ref)))
    return lins


def test_block_replay_sums_add_over_linears_and_transform_helps_outliers():
    lins = _block(40, 64, [(96, 256), (128, 128)], ("scaled", 4, 20.0))
    (s, n_off), (s2, n_on) = oracle.block_replay_sums(lins)
    assert s == s2 and s > 0 and n_off > 0 and n_on > 0
    parts = [oracle.block_replay_sums([l]) for l in lins]
    assert abs(sum(p[0][0] for p in parts) - s) <= 1e-9 * s
    assert abs(sum(p[0][1] for p in parts) - n_off) <= 1e-9 * n_off
    assert abs(sum(p[1][1] for p in parts) - n_on) <= 1e-9 * n_on
    # the page's reason for the ON path: outlier channels hurt plain MXFP4 more
    assert oracle.sqnr_db(s, n_on) > oracle.sqnr_db(s, n_off)


def test_block_replay_of_exact_block_has_no_noise():
    """A block whose activations and weights are exactly representable in MXFP4 (one value per
    block and power-of-two scales) and whose BF16 product is exact: OFF has zero noise."""
    x = np.full((8, 128), 0x3F80, np.uint16)   # 1.0
    w = np.full((16, 128), 0x3F00, np.uint16)  # 0.5
    y_ref = oracle.bf16_bits_to_f64(x) @ oracle.bf16_bits_to_f64(w).T  # 64 exactly
    (s, n_off), _ = oracle.block_replay_sums([(x, w, y_ref)])
    assert n_off == 0.0 and s == 8 * 16 * 64.0 ** 2
