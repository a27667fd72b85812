"""GPU parity: the gfx950 kernels (through the C ABI) against the CPU oracle.

Codes and scales must match byte for byte; GEMM outputs must satisfy
|y - y_ref| <= 2^-7 |y_ref| + 1e-3 rms(y_ref) with y_ref the oracle's float64
QDQ result computed from the oracle's own codes (identical to the GPU's).
"""

import sys

import numpy as np
import pytest
import torch

import mx_bit_quantized_amd as mxq
import oracle
import synth
from gpu_util import (W4A4_WAVE_KERNEL, assert_codes_equal, assert_output_close, code_rows, dev_bf16,
                      group_major_scales, host_bits, host_f32, host_u8, sample_rows, w4a4_waves)

# (mode, waves): the pipelined W4A4 GEMM with one and with two waves per SIMD, W4A8
PIPE_KINDS = [(mxq.W4A4, 4), (mxq.W4A4, 8), (mxq.W4A8, 4)]


def _pipe_kernel_check(mode, waves, m, n, k):
    name = mxq.gemm_kernel_name(mode, m, n, k)
    assert name.startswith("pipe_"), name
    if mode == mxq.W4A4:
        assert name == W4A4_WAVE_KERNEL[waves], name

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


def _bits(x):
    return synth.f32_to_bf16_bits(np.asarray(x, np.float32))


def _edge_activation(m, k, seed):
    g = np.random.default_rng(seed)
    x = synth.activation_bf16(seed, m, k, ("student_t",))
    if m >= 8:
        x[1] = 0                                                   # all-zero row
        x[2, : min(k, 64)] = 0                                     # zero blocks
        x[3] = (g.integers(0, 0x80, k) | (g.integers(0, 2, k) << 15)).astype(np.uint16)  # subnormals
        x[4] = _bits(g.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], k) * g.choice([-1, 1], k))  # FP4 ties
        x[5, 7] = 0x8000
        x[6] = _bits(g.standard_normal(k) * 1e25)
    return x


# ---------------------------------------------------------------- quantizers

@pytest.mark.parametrize("n,k", [(512, 512), (40, 96), (1, 32), (300, 160)])
def test_weight_pack_bit_exact(n, k):
    say("weight_pack", n, k)
    w = synth.weight_bf16(1, n, k)
    w[0, :32] = 0
    codes, scales = mxq.quantize_weight_mxfp4(dev_bf16(w))
    torch.cuda.synchronize()
    want_c, want_s = oracle.mxfp4_quantize(w)
    assert_codes_equal(host_u8(scales), group_major_scales(want_s), "weight scales")
    assert_codes_equal(code_rows(codes, n, k, 4), want_c, "weight codes")


@pytest.mark.parametrize("mode", [mxq.W4A4, mxq.W4A8])
@pytest.mark.parametrize("m,k", [(256, 512), (37, 96), (8, 32), (130, 5120)])
def test_quantize_act_bit_exact(mode, m, k):
    say("quantize_act", mode, m, k)
    x = _edge_activation(m, k, 100 + m)
    codes, scales = mxq.quantize_act(mode, dev_bf16(x))
    torch.cuda.synchronize()
    want_c, want_s = oracle.quantize_act(mode, x)
    if mode == mxq.W4A4:
        assert_codes_equal(host_u8(scales), group_major_scales(want_s), "mxfp4 scales")
    else:
        assert_codes_equal(host_f32(scales).view(np.uint32), want_s.view(np.uint32), "fp8 scales")
    got_c = code_rows(codes, m, k, 4) if mode == mxq.W4A4 else host_u8(codes)
    assert_codes_equal(got_c, want_c, "act codes")


# -------------------------------------------------------------------- GEMM

def _gemm_case(mode, m, n, k, seed, epilogue=mxq.EPI_NONE, bias=False):
    x = _edge_activation(m, k, seed)
    w = synth.weight_bf16(seed, n, k)
    b = _bits(np.random.default_rng(seed).standard_normal(n) * 0.1) if bias else None
    wc, ws = mxq.quantize_weight_mxfp4(dev_bf16(w))
    ac, asc = mxq.quantize_act(mode, dev_bf16(x))
    y = mxq.gemm(mode, ac, asc, wc, ws, dev_bf16(b) if bias else None, epilogue)
    torch.cuda.synchronize()
    owc, ows = oracle.mxfp4_quantize(w)
    oac, oas = oracle.quantize_act(mode, x)
    bias64 = oracle.bf16_bits_to_f64(b) if bias else None
    y_ref = oracle.qdq_matmul(mode, oac, oas, owc, ows, bias64, epilogue)
    return host_bits(y), y_ref


@pytest.mark.parametrize("mode", [mxq.W4A4, mxq.W4A8])
@pytest.mark.parametrize("m,n,k", [(256, 512, 512), (1, 64, 256), (37, 40, 96), (200, 100, 32),
                                   (129, 257, 1056), (64, 128, 5120)])
def test_gemm_matches_oracle(mode, m, n, k):
    say("gemm", mode, m, n, k)
    y, y_ref = _gemm_case(mode, m, n, k, seed=m * 7 + n)
    assert_output_close(y, y_ref, f"gemm mode={mode} {m}x{n}x{k}")


# Shapes that take the LDS-pipelined persistent kernel: exactly one ring of
# stages (4 for W4A4, more than the W4A8 ring), stage counts that are not
# multiples of the ring depth (the ring slot rotates from tile to tile),
# partial M and N tiles, a full A14B-width K, and grids with more tiles than
# CUs, so that workgroups walk several tiles and the copies run across tile
# boundaries (2250 x 7424: 261 tiles, not a multiple of 8; 4352 x 4096: 272).
PIPE_SHAPES = [(256, 256, 512), (300, 264, 640), (600, 512, 512), (257, 768, 1024), (512, 256, 5120),
               (1000, 1280, 896), (2250, 7424, 512), (4352, 4096, 640)]


@pytest.mark.parametrize("mode,waves", PIPE_KINDS)
@pytest.mark.parametrize("m,n,k", PIPE_SHAPES)
def test_gemm_pipelined_kernel_matches_oracle(mode, waves, m, n, k):
    say("gemm pipe", mode, waves, m, n, k)
    with w4a4_waves(waves):
        _pipe_kernel_check(mode, waves, m, n, k)
        y, y_ref = _gemm_case(mode, m, n, k, seed=m + 3 * n + k)
    assert_output_close(y, y_ref, f"gemm pipe mode={mode} waves={waves} {m}x{n}x{k}")


# The fewest stages the pipelined kernel takes: as many as its ring holds (W4A4
# four stages of 128 elements, W4A8 three), so the copy ring wraps inside
# every tile and the waits of the first stages overlap the previous tile's.
@pytest.mark.parametrize("mode,waves,m,n,k", [(mxq.W4A4, 4, 700, 2048, 512), (mxq.W4A4, 8, 700, 2048, 512),
                                              (mxq.W4A4, 8, 4352, 4096, 512), (mxq.W4A8, 4, 256, 512, 384),
                                              (mxq.W4A8, 4, 700, 2048, 384), (mxq.W4A8, 4, 4352, 4096, 384)])
def test_gemm_pipelined_at_the_fewest_stages(mode, waves, m, n, k):
    say("gemm pipe fewest stages", mode, waves, m, n, k)
    with w4a4_waves(waves):
        _pipe_kernel_check(mode, waves, m, n, k)
        assert not mxq.gemm_kernel_name(mode, m, n, k - 128).startswith("pipe_")
        y, y_ref = _gemm_case(mode, m, n, k, seed=7 * m + n + k)
    assert_output_close(y, y_ref, f"gemm pipe fewest stages mode={mode} waves={waves} {m}x{n}x{k}")


# Each combination of bias and GELU is a kernel of its own (the one without
# either is covered above).
@pytest.mark.parametrize("mode,waves", PIPE_KINDS)
@pytest.mark.parametrize("m,n,k", [(300, 512, 640), (4352, 4096, 640)])
@pytest.mark.parametrize("epilogue,bias", [(mxq.EPI_GELU_TANH, True), (mxq.EPI_NONE, True),
                                           (mxq.EPI_GELU_TANH, False)])
def test_gemm_pipelined_bias_and_gelu(mode, waves, m, n, k, epilogue, bias):
    say("gemm pipe epilogue", mode, waves, m, n, k, epilogue, bias)
    with w4a4_waves(waves):
        _pipe_kernel_check(mode, waves, m, n, k)
        y, y_ref = _gemm_case(mode, m, n, k, seed=8, epilogue=epilogue, bias=bias)
    assert_output_close(y, y_ref, f"pipe epilogue={epilogue} bias={bias} waves={waves} {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(300, 512, 640), (2250, 7424, 512), (4352, 4096, 640)])
def test_gemm_w4a4_four_and_eight_waves_bit_identical(m, n, k):
    """Both W4A4 kernels take the same MFMAs in the same order over K: equal bits."""
    say("gemm 4 vs 8 waves", m, n, k)
    x = dev_bf16(_edge_activation(m, k, 5 * m))
    wc, ws = mxq.quantize_weight_mxfp4(dev_bf16(synth.weight_bf16(9, n, k)))
    ac, asc = mxq.quantize_act(mxq.W4A4, x)
    b = dev_bf16(_bits(np.random.default_rng(m).standard_normal(n) * 0.1))
    outs = {}
    for waves in (4, 8):
        with w4a4_waves(waves):
            _pipe_kernel_check(mxq.W4A4, waves, m, n, k)
            outs[waves] = (mxq.gemm(mxq.W4A4, ac, asc, wc, ws, b, mxq.EPI_GELU_TANH),
                           mxq.gemm_mxfp4_out(ac, asc, wc, ws, b, mxq.EPI_GELU_TANH))
    torch.cuda.synchronize()
    assert torch.equal(outs[4][0], outs[8][0])
    assert torch.equal(outs[4][1][0], outs[8][1][0]) and torch.equal(outs[4][1][1], outs[8][1][1])


@pytest.mark.parametrize("mode", [mxq.W4A4, mxq.W4A8])
def test_gemm_bias_and_gelu_epilogue(mode):
    say("gemm epilogue", mode)
    y, y_ref = _gemm_case(mode, 96, 192, 512, seed=5, epilogue=mxq.EPI_GELU_TANH, bias=True)
    assert_output_close(y, y_ref, "bias+gelu")


def test_gemm_identity_weight_reproduces_dequantized_activations():
    """W = I is exact in MXFP4, so y must equal bf16(DQ(Q(x))) (checked within tolerance, per element)."""
    say("gemm identity")
    k = 256
    eye = _bits(np.eye(k))
    x = synth.activation_bf16(3, 64, k, ("scaled", 4, 20.0))
    for mode in (mxq.W4A4, mxq.W4A8):
        wc, ws = mxq.quantize_weight_mxfp4(dev_bf16(eye))
        ac, asc = mxq.quantize_act(mode, dev_bf16(x))
        y = host_bits(mxq.gemm(mode, ac, asc, wc, ws))
        oac, oas = oracle.quantize_act(mode, x)
        assert_output_close(y, oracle.dequantize_act(mode, oac, oas), f"identity mode={mode}")


def test_gemm_empty_is_noop():
    say("gemm empty")
    wc = torch.zeros((64, 128), dtype=torch.uint8, device="cuda")
    ws = torch.full((2, 64, 4), 127, dtype=torch.uint8, device="cuda")
    ac = torch.zeros((0, 128), dtype=torch.uint8, device="cuda")
    asc = torch.zeros((2, 0, 4), dtype=torch.uint8, device="cuda")
    y = mxq.gemm(mxq.W4A4, ac, asc, wc, ws)
    assert y.shape == (0, 64)


# ----------------------------------------------------------------- qlinear

def test_config1_qlinear_both_modes_through_policy():
    """Config 1: X [256x512] with 4 outlier channels x20, W [512x512], once W4A4 and once W4A8."""
    wl = synth.workload(1)
    say("config1")
    x = synth.activation_bf16(1, 256, 512, wl.outliers)
    w = synth.weight_bf16(1, 512, 512)
    policy = mxq.Policy(wl.policy())
    wc, ws = mxq.quantize_weight_mxfp4(dev_bf16(w))
    xd = dev_bf16(x)
    owc, ows = oracle.mxfp4_quantize(w)
    assert_codes_equal(code_rows(wc, 512, 512, 4), owc, "config1 weight codes")
    assert_codes_equal(host_u8(ws), group_major_scales(ows), "config1 weight scales")
    for block in range(2):
        mode = policy.mode(0, block)
        assert mode == oracle.policy_mode(wl.policy(), 0, block)
        ws_bytes = mxq.qlinear_workspace_bytes(mode, 256, 512)
        work = torch.empty((ws_bytes,), dtype=torch.uint8, device="cuda")
        y = mxq.qlinear(policy, 0, block, xd, wc, ws, workspace=work)
        torch.cuda.synchronize()
        y_ref, oac, oas = oracle.qlinear(mode, x, owc, ows)
        # the workspace holds the activation codes the GEMM consumed
        codes_len = oac.size
        got = code_rows(work[:codes_len], 256, 512, 4) if mode == mxq.W4A4 else host_u8(work[:codes_len]).reshape(oac.shape)
        assert_codes_equal(got, oac, f"config1 act codes mode={mode}")
        assert_output_close(host_bits(y), y_ref, f"config1 mode={mode}")
    policy.close()


def test_qlinear_rejects_policy_modes_without_writing():
    say("qlinear reject")
    y = torch.full((4, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mxq.MxqError):
        mxq.Policy([[mxq.POLICY_BF16]])
    p = mxq.Policy([[mxq.W4A4]])
    with pytest.raises(mxq.MxqError):
        mxq.qlinear(p, 0, 1, torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda"),
                    torch.zeros((64, 32), dtype=torch.uint8, device="cuda"),
                    torch.zeros((1, 64, 4), dtype=torch.uint8, device="cuda"), y=y)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


def test_determinism_byte_identical_reruns():
    say("determinism")
    x = dev_bf16(synth.activation_bf16(11, 300, 1024, ("student_t",)))
    wc, ws = mxq.quantize_weight_mxfp4(dev_bf16(synth.weight_bf16(11, 640, 1024)))
    outs = []
    for _ in range(2):
        for mode in (mxq.W4A4, mxq.W4A8):
            ac, asc = mxq.quantize_act(mode, x)
            outs.append(host_bits(mxq.gemm(mode, ac, asc, wc, ws)))
    assert np.array_equal(outs[0], outs[2]) and np.array_equal(outs[1], outs[3])
