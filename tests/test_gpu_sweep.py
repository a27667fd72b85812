"""Seeded random-shape sweep of the GEMM paths against the oracle (GPU).

Each case draws its shape and options from a fixed seed: M (ragged against
the 256-row tiles), N (a multiple of 8, ragged against 256-column tiles), K
(a multiple of 128 for the pipelined kernel, or any multiple of 32 for the
direct one), mode, epilogue, bias and the W4A4 wave count. Checks:

* activation codes and scales equal the oracle's byte for byte;
* the bf16 output is within the output tolerance of the oracle's QDQ result
  on every element (the shapes are small enough for the full product);
* where the shape allows them, the fused MXFP4, transformed-MXFP4 and static
  FP8 outputs equal the plain GEMM followed by the matching quantizer (the
  static scale calibrated on that GEMM's output), byte for byte;
* on the pipelined W4A4 shapes, the GEMM with SVDQuant's low-rank branch (a
  seeded rank of 32 to 128) is within the output tolerance of the oracle on
  every element, and its MXFP4 output equals the quantizer applied to its
  bf16 output.
"""

import sys

import numpy as np
import pytest
import torch

import mx_bit_quantized_amd as mxq
import oracle
import synth
from gpu_util import assert_codes_equal, assert_output_close, dev_bf16, host_bits, host_u8, w4a4_waves

pytestmark = pytest.mark.gpu

N_CASES = 48


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    mxq.lib()
    yield
    torch.cuda.synchronize()


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _draw(case):
    g = np.random.default_rng(1000 + case)
    pipelined = case % 4 != 3  # every fourth case may take the direct kernel
    m = int(g.integers(256, 1800)) if pipelined else int(g.integers(1, 600))
    mode = int(g.integers(0, 2)) if pipelined else (case // 4) % 2
    # half the pipelined cases take N in whole 128-column panels (W4A4) or in
    # multiples of 32 (W4A8), the shapes of the fused MXFP4 and static FP8
    # outputs
    if pipelined and case % 2 == 0:
        n = 128 * int(g.integers(2, 26)) if mode == 0 else 32 * int(g.integers(8, 100))
    else:
        n = 8 * int(g.integers(32, 400))
    k = 128 * int(g.integers(4, 24)) if pipelined else 32 * int(g.integers(1, 80))
    if mode == mxq.W4A8 and pipelined:
        k = max(k, 384)  # the W4A8 ring holds three stages
    epilogue = int(g.integers(0, 2))
    bias = bool(g.integers(0, 2))
    waves = int(g.choice([4, 8]))
    return m, n, k, mode, epilogue, bias, waves


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_shape_matches_oracle(case):
    m, n, k, mode, epilogue, bias, waves = _draw(case)
    say("sweep", case, dict(m=m, n=n, k=k, mode=mode, epi=epilogue, bias=bias, waves=waves))
    x = synth.activation_bf16(3000 + case, m, k, ("student_t",))
    w = synth.weight_bf16(4000 + case, n, k)
    b = synth.f32_to_bf16_bits((np.random.default_rng(case).standard_normal(n) * 0.1).astype(np.float32)) \
        if bias else None
    with w4a4_waves(waves):
        name = mxq.gemm_kernel_name(mode, m, n, k)
        wc, ws = mxq.quantize_weight_mxfp4(dev_bf16(w))
        ac, asc = mxq.quantize_act(mode, dev_bf16(x))
        bd = dev_bf16(b) if bias else None
        y = mxq.gemm(mode, ac, asc, wc, ws, bd, epilogue)
        torch.cuda.synchronize()
    say("kernel", name)
    oac, oas = oracle.quantize_act(mode, x)
    if mode == mxq.W4A4:
        c_rm, s_rm = mxq.mxfp4_to_canonical(ac, asc, m, k)
        torch.cuda.synchronize()
        assert_codes_equal(host_u8(c_rm), oac, f"case {case} activation codes")
        assert_codes_equal(host_u8(s_rm), oas, f"case {case} activation scales")
    else:
        assert_codes_equal(host_u8(ac), oac, f"case {case} FP8 codes")
        got_s = asc.cpu().numpy().view(np.uint32)
        assert np.array_equal(got_s, np.asarray(oas, np.float32).view(np.uint32)), f"case {case} FP8 scales"
    owc, ows = oracle.mxfp4_quantize(w)
    b64 = oracle.bf16_bits_to_f64(b) if bias else None
    y_ref = oracle.qdq_matmul(mode, oac, oas, owc, ows, b64, epilogue)
    assert_output_close(host_bits(y), y_ref, f"case {case} {name} [{m}x{n}x{k}]")

    if mode == mxq.W4A4 and mxq.gemm_mxfp4_out_supported(m, n, k):
        with w4a4_waves(waves):
            fc, fs = mxq.gemm_mxfp4_out(ac, asc, wc, ws, bd, epilogue)
            rc, rs = mxq.quantize_act(mxq.W4A4, y)
            g = np.random.default_rng(case)
            mult = torch.from_numpy(((g.random(n) + 0.5) * 0.088).astype(np.float32)).to("cuda:0")
            hc, hs = mxq.gemm_mxfp4_hadamard_out(ac, asc, wc, ws, mult, bd, epilogue)
            tc, ts = mxq.quantize_mxfp4_hadamard(y, mult)
            torch.cuda.synchronize()
        assert torch.equal(fc, rc) and torch.equal(fs, rs), f"case {case}: fused MXFP4 output differs"
        assert torch.equal(hc, tc) and torch.equal(hs, ts), f"case {case}: fused transformed output differs"

    if mode == mxq.W4A4 and mxq.gemm_lowrank_supported(m, n, k):
        # SVDQuant's branch in the GEMM's sums: a seeded rank and factors
        gr = np.random.default_rng(5000 + case)
        r = int(gr.choice([32, 64, 96, 128]))
        t = synth.f32_to_bf16_bits((gr.standard_normal((m, r)) * 0.5).astype(np.float32))
        l2 = synth.f32_to_bf16_bits((gr.standard_normal((n, r)) * 0.05).astype(np.float32))
        with w4a4_waves(waves):
            yl = mxq.gemm_lowrank(ac, asc, wc, ws, dev_bf16(t), dev_bf16(l2), bd, epilogue)
            torch.cuda.synchronize()
        want = oracle.svdquant_linear_fused(mxq.W4A4, oac, oas, owc, ows, t, l2, b64, epilogue)
        assert_output_close(host_bits(yl), want, f"case {case} gemm+branch r={r} [{m}x{n}x{k}]")
        if mxq.gemm_lowrank_supported(m, n, k, mxfp4_out=True):
            with w4a4_waves(waves):
                lc, ls = mxq.gemm_lowrank(ac, asc, wc, ws, dev_bf16(t), dev_bf16(l2), bd, epilogue, mxfp4_out=True)
                qc, qs = mxq.quantize_act(mxq.W4A4, yl)
                torch.cuda.synchronize()
            assert torch.equal(lc, qc) and torch.equal(ls, qs), f"case {case}: fused branch MXFP4 output differs"

    if mode == mxq.W4A8 and mxq.gemm_fp8_static_out_supported(m, n, k):
        amax = mxq.fp8_calibrate(y)
        rc, rs = mxq.quantize_act_fp8_static(y, amax)
        fc, fs = mxq.gemm_fp8_static_out(ac, asc, wc, ws, amax, bd, epilogue)
        torch.cuda.synchronize()
        assert torch.equal(fc, rc) and torch.equal(fs, rs), f"case {case}: fused static FP8 output differs"


def test_sweep_covers_both_kernels_modes_and_options():
    draws = [_draw(c) for c in range(N_CASES)]
    kinds = {(mxq.gemm_kernel_name(md, m, n, k).split("_")[0], md) for m, n, k, md, *_ in draws}
    assert kinds == {("pipe", 0), ("pipe", 1), ("direct", 0), ("direct", 1)}
    assert {d[3] for d in draws} == {0, 1} and {d[4] for d in draws} == {0, 1} and {d[5] for d in draws} == {False, True}
    assert any(d[0] % 256 for d in draws) and any(d[1] % 256 for d in draws)
    assert sum(1 for d in draws if d[3] == 0 and mxq.gemm_mxfp4_out_supported(d[0], d[1], d[2])) >= 3
    assert sum(1 for d in draws if d[3] == 1 and mxq.gemm_fp8_static_out_supported(d[0], d[1], d[2])) >= 3
