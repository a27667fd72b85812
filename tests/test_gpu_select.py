"""GPU parity of the calibration-driven block selection: the SQNR energy
reduction, the native block replay (OFF = plain MXFP4, ON = transform_on) and
the policy it yields, against the CPU oracle.

The replay's codes are the oracle's bit for bit; its bf16 outputs differ from
the oracle's bf16 rounding of the float64 QDQ result only where the fp32
accumulation lands on the other side of a rounding boundary, so the noise
energies agree to a few parts in a thousand and the SQNRs to a few thousandths
of a dB. The captured BF16 outputs are the oracle's: float64 products rounded
to bf16.
"""

import math
import sys

import numpy as np
import pytest
import torch

import mx_bit_quantized_amd as mxq
import oracle
import synth
from gpu_util import dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    mxq.lib()
    yield
    torch.cuda.synchronize()


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _sums():
    return torch.zeros((2,), dtype=torch.float64, device="cuda:0")


@pytest.mark.parametrize("n", [1, 7, 8, 1000, 4099, 1 << 20])
def test_sqnr_accumulate_matches_oracle(n):
    say("sqnr sums", n)
    g = np.random.default_rng(n)
    r = synth.f32_to_bf16_bits((g.standard_normal(n) * np.ldexp(1.0, g.integers(-20, 20, n))).astype(np.float32))
    y = synth.f32_to_bf16_bits((oracle.bf16_bits_to_f32(r) * (1 + 0.05 * g.standard_normal(n))).astype(np.float32))
    sums = _sums()
    mxq.sqnr_accumulate(dev_bf16(y), dev_bf16(r), sums)
    mxq.sqnr_accumulate(dev_bf16(y), dev_bf16(r), sums)  # folds
    torch.cuda.synchronize()
    s, e = oracle.sqnr_sums(oracle.bf16_bits_to_f64(y), oracle.bf16_bits_to_f64(r))
    got = sums.cpu().numpy()
    assert abs(got[0] - 2 * s) <= 1e-12 * 2 * s
    assert abs(got[1] - 2 * e) <= 1e-12 * 2 * e


def _block(seed, m, dims, outliers, w_scale=1.0):
    lins = []
    for i, (n, k) in enumerate(dims):
        x = synth.activation_bf16(seed + i, m, k, outliers)
        w = synth.weight_bf16(seed + i, n, k)
        if w_scale != 1.0:
            w = synth.f32_to_bf16_bits(oracle.bf16_bits_to_f32(w) * np.float32(w_scale))
        y_ref = oracle.f64_to_bf16_bits(oracle.bf16_bits_to_f64(x) @ oracle.bf16_bits_to_f64(w).T)
        lins.append((x, w, y_ref))
    return lins


def _exact_block(m, n, k, seed):
    """Activations and weights exactly representable in MXFP4 with an exact bf16 product."""
    g = np.random.default_rng(seed)
    x = synth.f32_to_bf16_bits(g.choice([-2.0, -1.0, 1.0, 2.0], (m, k)).astype(np.float32))
    w = synth.f32_to_bf16_bits(g.choice([-0.5, 0.5], (n, k)).astype(np.float32))
    y_ref = oracle.f64_to_bf16_bits(oracle.bf16_bits_to_f64(x) @ oracle.bf16_bits_to_f64(w).T)
    return [(x, w, y_ref)]


def _floor_block(m, n, k, seed):
    """Below every floor: each 32-block of x carries one element 1000 times larger, on a weight
    column of zeros, so MXFP4 (one scale per block) flushes the elements that make the output."""
    g = np.random.default_rng(seed)
    x = g.standard_normal((m, k)).astype(np.float32)
    x[:, ::32] *= np.float32(1000.0)
    w = (g.standard_normal((n, k)) * 0.02).astype(np.float32)
    w[:, ::32] = 0
    xb, wb = synth.f32_to_bf16_bits(x), synth.f32_to_bf16_bits(w)
    y_ref = oracle.f64_to_bf16_bits(oracle.bf16_bits_to_f64(xb) @ oracle.bf16_bits_to_f64(wb).T)
    return [(xb, wb, y_ref)]


def _gpu_replay(lins):
    dev = [(dev_bf16(x), dev_bf16(w), dev_bf16(y)) for x, w, y in lins]
    s_off, s_on = _sums(), _sums()
    mxq.block_replay_sqnr(dev, s_off, s_on)
    torch.cuda.synchronize()
    return s_off.cpu().numpy(), s_on.cpu().numpy()


def _oracle_replay(lins):
    return oracle.block_replay_sums([(x, w, oracle.bf16_bits_to_f64(y)) for x, w, y in lins])


@pytest.mark.parametrize("case", ["gauss", "outliers", "mixed_shapes"])
def test_block_replay_matches_oracle(case):
    say("block replay", case)
    if case == "gauss":
        lins = _block(10, 256, [(512, 512)], None)
    elif case == "outliers":
        lins = _block(20, 300, [(256, 384), (384, 256)], ("scaled", 4, 20.0))
    else:
        lins = _block(30, 100, [(264, 128), (128, 640), (96, 256)], ("student_t",))
    g_off, g_on = _gpu_replay(lins)
    (s, e_off), (_, e_on) = _oracle_replay(lins)
    assert abs(g_off[0] - s) <= 1e-12 * s and abs(g_on[0] - s) <= 1e-12 * s
    assert abs(g_off[1] - e_off) <= 5e-3 * e_off, (g_off[1], e_off)
    assert abs(g_on[1] - e_on) <= 5e-3 * e_on, (g_on[1], e_on)
    assert abs(oracle.sqnr_db(*g_off) - oracle.sqnr_db(s, e_off)) < 0.03
    assert abs(oracle.sqnr_db(*g_on) - oracle.sqnr_db(s, e_on)) < 0.03


def test_exact_block_has_no_off_noise():
    say("exact block")
    lins = _exact_block(64, 128, 256, 5)
    g_off, g_on = _gpu_replay(lins)
    assert g_off[1] == 0.0 and g_on[1] > 0.0
    assert oracle.sqnr_db(*g_off) == math.inf


def test_selector_policy_matches_oracle():
    """A small two-expert model of synthetic blocks with a spread of SQNRs: the GPU replay plus the
    library's rule ladder give the oracle's policy artifact for every tier."""
    say("selector policy")
    specs = [
        ("exact", None), ("gauss", None), ("t", ("student_t",)), ("heavy", ("scaled", 8, 60.0)),
        ("floor", None), ("s4x20", ("scaled", 4, 20.0)),
    ]
    n_exp, n_blk = 2, len(specs)
    s_off = np.zeros((n_exp, n_blk, 2))
    s_on = np.zeros((n_exp, n_blk, 2))
    o_off = np.zeros((n_exp, n_blk))
    o_on = np.zeros((n_exp, n_blk))
    for e in range(n_exp):
        for b, (kind, outl) in enumerate(specs):
            seed = 1000 + 37 * e + 5 * b
            if kind == "exact":
                lins = _exact_block(64, 96, 256, seed)
            elif kind == "floor":
                lins = _floor_block(128, 128, 256, seed)
            else:
                lins = _block(seed, 128, [(128, 256)], outl)
            g_off, g_on = _gpu_replay(lins)
            s_off[e, b], s_on[e, b] = g_off, g_on
            (s, eo), (_, en) = _oracle_replay(lins)
            o_off[e, b], o_on[e, b] = oracle.sqnr_db(s, eo), oracle.sqnr_db(s, en)
    for tier, name in ((mxq.TIER_LOW, "low"), (mxq.TIER_MID, "mid"), (mxq.TIER_HIGH, "high")):
        floor, w4a8, margin = oracle.TIERS[name]
        # no oracle value sits within 0.05 dB of a boundary, so the comparison is meaningful
        best = np.maximum(o_off, o_on)
        fin = np.isfinite(best)
        assert np.all(np.abs(best[fin] - floor) > 0.05) and np.all(np.abs(best[fin] - w4a8) > 0.05)
        diff = o_on - o_off
        fd = np.isfinite(diff) & (best >= w4a8)  # the margin rule is reached only there
        assert np.all(np.abs(diff[fd] - margin) > 0.05)
        got = mxq.policy_select(s_off, s_on, tier)
        want = oracle.select_policy(o_off, o_on, name)
        assert np.array_equal(got, want), (name, got, want, o_off, o_on)
        # the synthetic model yields more than one decision: bf16, W4A8 and W4A4 all occur
        assert {oracle.BF16_MODE, oracle.W4A8, oracle.W4A4} <= set(np.unique(want).tolist())
    say("sqnr off", np.round(o_off, 2).tolist(), "on", np.round(o_on, 2).tolist())
