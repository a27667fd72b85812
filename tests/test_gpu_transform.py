"""GPU parity of the transform_on mode (fixed block Hadamard rotation + SmoothQuant
ahead of MXFP4) against the CPU oracle.

The rotation's butterflies, the channel factors and the bf16 rounding are fp32
steps in a fixed order on both sides, so codes, scales, calibration maxima and
factors must match bit for bit; GEMM outputs within
|y - y_ref| <= 2^-7 |y_ref| + 1e-3 rms(y_ref).
"""

import sys

import numpy as np
import pytest
import torch

import mx_bit_quantized_amd as mxq
import oracle
import synth
from gpu_util import (assert_codes_equal, assert_output_close, code_rows, dev_bf16, group_major_scales, host_bits,
                      host_f32, host_u8, sample_rows)

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


def _f32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda:0")


def _bits32(t):
    return host_f32(t).view(np.uint32)


def _edge_rows(m, k, seed):
    g = np.random.default_rng(seed)
    x = synth.activation_bf16(seed, m, k, ("student_t",))
    if m >= 6:
        x[1] = 0
        x[2] = (g.integers(0, 0x80, k) | (g.integers(0, 2, k) << 15)).astype(np.uint16)  # subnormals
        x[3] = synth.f32_to_bf16_bits((g.standard_normal(k) * 1e30).astype(np.float32))
        x[4, ::7] = 0x8000
        x[5] = synth.f32_to_bf16_bits(g.integers(-8, 8, k).astype(np.float32))  # exact sums, many ties
    return x


def _factors(seed, k):
    g = np.random.default_rng(seed)
    ax = np.ldexp(g.uniform(1, 2, k), g.integers(-8, 8, k)).astype(np.float32)
    aw = np.ldexp(g.uniform(1, 2, k), g.integers(-12, -2, k)).astype(np.float32)
    ax[::17] = 0
    return oracle.smoothquant_factors(ax, aw)


def _check_quant(x, mult, what, ld=None):
    m, k = x.shape
    if ld is None:
        xd = dev_bf16(x)
        codes, scales = mxq.quantize_mxfp4_hadamard(xd, _f32_dev(mult))
    else:
        wide = np.zeros((m, ld), np.uint16)
        wide[:, :k] = x
        wide[:, k:] = 0x7F7F  # outside the rows: would change every block it reached
        xd = dev_bf16(wide)
        codes, scales = mxq.act_buffers(mxq.W4A4, m, k, "cuda:0")
        md = _f32_dev(mult)
        st = mxq.lib().mxq_quantize_mxfp4_hadamard(mxq._dev_ptr(xd, "x"), m, k, ld, mxq._dev_ptr(md, "mult"),
                                                    mxq._dev_ptr(codes, "c"), mxq._dev_ptr(scales, "s"),
                                                    mxq._stream_handle())
        assert st == mxq.OK
    torch.cuda.synchronize()
    want_c, want_s = oracle.mxfp4_quantize_hadamard(x, mult)
    assert_codes_equal(host_u8(scales), group_major_scales(want_s), f"{what} scales")
    assert_codes_equal(code_rows(codes, m, k, 4), want_c, f"{what} codes")


@pytest.mark.parametrize("m,k,ld", [(1, 128, None), (37, 384, None), (256, 5120, None), (130, 13824, None),
                                    (6, 256, 264), (1000, 640, None)])
def test_hadamard_quantizer_bit_exact(m, k, ld):
    say("hadamard quant", m, k, ld)
    x = _edge_rows(m, k, 500 + m)
    act_mult, w_mult = _factors(600 + k, k)
    _check_quant(x, act_mult, f"[{m}x{k}] act_mult", ld)
    _check_quant(x, w_mult, f"[{m}x{k}] w_mult", ld)
    _check_quant(x, np.full(k, oracle.INV_SQRT_BLOCK, np.float32), f"[{m}x{k}] rotation only", ld)


def test_hadamard_channel_amax_bit_exact():
    say("hadamard channel amax")
    batches = [_edge_rows(300, 512, 71), synth.activation_bf16(72, 17, 512, ("scaled", 4, 20.0)),
               synth.activation_bf16(73, 4099, 512, ("student_t",)), np.zeros((3, 512), np.uint16)]
    amax = torch.zeros((512,), dtype=torch.float32, device="cuda:0")
    for b in batches:
        mxq.hadamard_channel_amax(dev_bf16(b), amax)
    torch.cuda.synchronize()
    want = oracle.hadamard_channel_amax(batches)
    assert_codes_equal(_bits32(amax), want.view(np.uint32), "channel amax")
    # with a leading dimension
    m, k, ld = 40, 256, 384
    x = synth.activation_bf16(74, m, k, ("student_t",))
    wide = np.zeros((m, ld), np.uint16)
    wide[:, :k] = x
    wide[:, k:] = 0x7F7F
    a2 = torch.zeros((k,), dtype=torch.float32, device="cuda:0")
    wd = dev_bf16(wide)
    st = mxq.lib().mxq_hadamard_channel_amax(mxq._dev_ptr(wd, "x"), m, k, ld, mxq._dev_ptr(a2, "a"),
                                             mxq._stream_handle())
    assert st == mxq.OK
    torch.cuda.synchronize()
    assert_codes_equal(_bits32(a2), oracle.hadamard_channel_amax([x]).view(np.uint32), "channel amax ld")


def test_smoothquant_factors_bit_exact():
    say("smoothquant factors")
    g = np.random.default_rng(75)
    k = 14336
    ax = np.ldexp(g.uniform(1, 2, k), g.integers(-60, 60, k)).astype(np.float32)
    aw = np.ldexp(g.uniform(1, 2, k), g.integers(-60, 60, k)).astype(np.float32)
    ax[::13] = 0
    aw[::29] = 0
    am, wm = mxq.smoothquant_factors(_f32_dev(ax), _f32_dev(aw))
    torch.cuda.synchronize()
    oam, owm = oracle.smoothquant_factors(ax, aw)
    assert_codes_equal(_bits32(am), oam.view(np.uint32), "act_mult")
    assert_codes_equal(_bits32(wm), owm.view(np.uint32), "w_mult")


def _calibrated(x, w):
    """GPU calibration of one linear: rotated maxima, factors, transformed weight pack."""
    xd, wd = dev_bf16(x), dev_bf16(w)
    ax = mxq.hadamard_channel_amax(xd)
    aw = mxq.hadamard_channel_amax(wd)
    am, wm = mxq.smoothquant_factors(ax, aw)
    wc, ws = mxq.quantize_mxfp4_hadamard(wd, wm)
    return xd, am, wm, wc, ws


@pytest.mark.parametrize("m,n,k,epi", [(256, 512, 512, mxq.EPI_NONE), (512, 1024, 1024, mxq.EPI_GELU_TANH),
                                       (100, 264, 384, mxq.EPI_NONE)])
def test_transform_on_qlinear_through_policy(m, n, k, epi):
    say("transform qlinear", m, n, k, epi)
    x = synth.activation_bf16(80 + m, m, k, ("scaled", 4, 20.0))
    w = synth.weight_bf16(81 + m, n, k)
    xd, am, wm, wc, ws = _calibrated(x, w)
    policy = mxq.Policy([[mxq.POLICY_TRANSFORM_ON, mxq.W4A4]])
    y = mxq.qlinear_transform(policy, 0, 0, xd, wc, ws, am, None, epi)
    with pytest.raises(mxq.MxqError) as ei:
        mxq.qlinear(policy, 0, 0, xd, wc, ws, None, epi)
    assert ei.value.status == mxq.ERR_MODE
    torch.cuda.synchronize()
    policy.close()
    oam, owm = oracle.smoothquant_factors(oracle.hadamard_channel_amax([x]), oracle.hadamard_channel_amax([w]))
    assert_codes_equal(_bits32(am), oam.view(np.uint32), "act_mult")
    owc, ows = oracle.mxfp4_quantize_hadamard(w, owm)
    assert_codes_equal(code_rows(wc, n, k, 4), owc, "transformed weight codes")
    y_ref, _, _ = oracle.qlinear_transform(oracle.TRANSFORM_ON, x, owc, ows, oam, None, epi)
    assert_output_close(host_bits(y), y_ref, f"transform qlinear [{m}x{n}x{k}]")


def test_a14b_qkv_480p_transform_full_size():
    """A14B self-attention QKV at 480p (32760 x 5120 -> 15360) on transform_on: calibration on the
    whole activation and weight, the factor vectors and the transformed weight compared whole,
    activation codes and y on sampled rows and columns."""
    wl = synth.workload(2)
    lin = wl.linears[0]
    m, n, k = wl.m_video, lin.n, lin.k
    what = f"a14b qkv transform [{m}x{n}x{k}]"
    say(what)
    x = synth.activation_bf16(2, m, k, wl.outliers, tensor_id=synth.T_X_VIDEO)
    xd = dev_bf16(x)
    wd = synth.weight_bf16_device(2, n, k, 0, 0, 0)
    ax = mxq.hadamard_channel_amax(xd)
    aw = mxq.hadamard_channel_amax(wd)
    am, wm = mxq.smoothquant_factors(ax, aw)
    wc, ws = mxq.quantize_mxfp4_hadamard(wd, wm)
    codes, scales = mxq.quantize_mxfp4_hadamard(xd, am)
    y = mxq.gemm(mxq.W4A4, codes, scales, wc, ws)
    torch.cuda.synchronize()
    w_bits = host_bits(wd)
    del wd
    oax = oracle.hadamard_channel_amax([x])
    oaw = oracle.hadamard_channel_amax([w_bits])
    assert_codes_equal(_bits32(ax), oax.view(np.uint32), what + " act amax")
    assert_codes_equal(_bits32(aw), oaw.view(np.uint32), what + " weight amax")
    oam, owm = oracle.smoothquant_factors(oax, oaw)
    assert_codes_equal(_bits32(am), oam.view(np.uint32), what + " act_mult")
    assert_codes_equal(_bits32(wm), owm.view(np.uint32), what + " w_mult")
    rows = sample_rows(m, 24, 211)
    cols = sample_rows(n, 256, 212)
    owc, ows = oracle.mxfp4_quantize_hadamard(w_bits[cols], owm)
    assert_codes_equal(code_rows(wc, n, k, 4, cols), owc, what + " weight codes")
    oac, oas = oracle.mxfp4_quantize_hadamard(x[rows], oam)
    assert_codes_equal(code_rows(codes, m, k, 4, rows), oac, what + " act codes")
    y_ref = oracle.qdq_matmul(oracle.W4A4, oac, oas, owc, ows)
    idx = lambda a: torch.from_numpy(np.asarray(a, np.int64)).to("cuda:0")
    y_got = host_bits(y.index_select(0, idx(rows)).index_select(1, idx(cols)))
    rep = assert_output_close(y_got, y_ref, what)
    say(f"{what}: worst/bound {rep['worst_ratio']:.3f}")
