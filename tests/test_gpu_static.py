"""GPU parity of static (per-tensor) FP8 activations: calibration amax, the
static quantizer, and W4A8 GEMMs on its output, against the CPU oracle.

The page's format table calls the W4A8 activations FP8 E4M3 static; the scale
is fixed from a calibration amax (s = amax / 448), and values past it saturate.
Calibration maxima and codes must match the oracle bit for bit; GEMM outputs
within |y - y_ref| <= 2^-7 |y_ref| + 1e-3 rms(y_ref).
"""

import sys

import numpy as np
import pytest
import torch

import mx_bit_quantized_amd as mxq
import oracle
import synth
from gpu_util import assert_codes_equal, assert_output_close, dev_bf16, host_bits, host_f32, host_u8, sample_rows

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


def _amax_dev(v):
    return torch.tensor([float(np.float32(v))], dtype=torch.float32, device="cuda:0")


def _f32_bits(t):
    return host_f32(t).view(np.uint32)


def _check_static(x_bits, amax, what, ld=None):
    """Quantize x with a static amax on the GPU (optionally from a wider buffer) and compare with the oracle."""
    m, k = x_bits.shape
    if ld is None:
        xd = dev_bf16(x_bits)
    else:  # x as the first k columns of an [m, ld] buffer
        wide = np.zeros((m, ld), np.uint16)
        wide[:, :k] = x_bits
        wide[:, k:] = 0x7F7F  # past the row: would saturate every code if it were read
        xd = dev_bf16(wide)
    codes = torch.empty((m, k), dtype=torch.uint8, device="cuda:0")
    scales = torch.empty((m,), dtype=torch.float32, device="cuda:0")
    L = mxq.lib()
    st = L.mxq_quantize_act_fp8_static(mxq._dev_ptr(xd, "x"), m, k, ld or k, mxq._dev_ptr(_amax_dev(amax), "amax"),
                                       mxq._dev_ptr(codes, "codes"), mxq._dev_ptr(scales, "scales"),
                                       mxq._stream_handle())
    assert st == mxq.OK, st
    torch.cuda.synchronize()
    want_c, want_s = oracle.fp8_quantize_static(x_bits, np.float32(amax))
    assert_codes_equal(_f32_bits(scales), want_s.view(np.uint32), f"{what} scales")
    assert_codes_equal(host_u8(codes), want_c, f"{what} codes")


# ------------------------------------------------------------- quantizer ----

AMAX_SET = [448.0, 1.0, 3.296875, 0.0, 1e-44, 2.43e-17, 1e-30, 3.3895314e38, 65504.0, 5.27e-36, 0.7, 12345.678]


@pytest.mark.parametrize("amax", AMAX_SET)
def test_static_every_finite_bf16(amax):
    """All finite bf16 patterns, both signs, one static amax each (saturation, subnormal and
    pre-scaled divisors included)."""
    say("static all-bf16", amax)
    pos = np.arange(0, 0x7F80, dtype=np.uint32).astype(np.uint16)
    x = np.concatenate([pos, pos | 0x8000]).reshape(255, 256)
    _check_static(x, amax, f"all-bf16 amax={amax}")


@pytest.mark.parametrize("m,k,ld", [(1, 32, None), (3, 96, 104), (257, 5120, None), (64, 13824, None),
                                    (1000, 160, 192), (4097, 32, None)])
def test_static_shapes(m, k, ld):
    say("static shapes", m, k, ld)
    x = synth.activation_bf16(900 + m, m, k, ("student_t",))
    true_amax = float(np.abs(oracle.bf16_bits_to_f64(x)).max())
    for frac in (1.0, 0.05, 3.0):
        _check_static(x, true_amax * frac, f"[{m}x{k} ld={ld}] amax x{frac}", ld)


# ----------------------------------------------------------- calibration ----

def test_calibration_amax_matches_oracle_and_folds():
    say("calibrate")
    batches = [synth.activation_bf16(950, 300, 512, ("student_t",)),
               synth.activation_bf16(951, 17, 96, ("scaled", 4, 20.0)),
               synth.activation_bf16(952, 4097, 64, ("student_t",)),
               np.zeros((5, 32), np.uint16)]
    batches[3][2, 3] = 0x8000
    amax = torch.zeros((1,), dtype=torch.float32, device="cuda:0")
    for b in batches:
        mxq.fp8_calibrate(dev_bf16(b), amax)
        torch.cuda.synchronize()
    want = oracle.fp8_calibration_amax(batches)
    assert _f32_bits(amax)[0] == np.float32(want).view(np.uint32), (host_f32(amax)[0], want)
    # any order gives the same maximum; a zero batch alone gives 0
    rev = torch.zeros((1,), dtype=torch.float32, device="cuda:0")
    for b in batches[::-1]:
        mxq.fp8_calibrate(dev_bf16(b), rev)
    z = mxq.fp8_calibrate(dev_bf16(batches[3]))
    torch.cuda.synchronize()
    assert _f32_bits(rev)[0] == _f32_bits(amax)[0]
    assert host_f32(z)[0] == 0.0
    # a running maximum above every element stays as it is
    big = _amax_dev(1e30)
    mxq.fp8_calibrate(dev_bf16(batches[0]), big)
    torch.cuda.synchronize()
    assert host_f32(big)[0] == np.float32(1e30)


def test_calibration_with_leading_dimension():
    say("calibrate ld")
    m, k, ld = 40, 96, 128
    x = synth.activation_bf16(953, m, k, ("student_t",))
    wide = np.zeros((m, ld), np.uint16)
    wide[:, :k] = x
    wide[:, k:] = 0x7F7F  # outside the rows: must not count
    xd = dev_bf16(wide)
    amax = torch.zeros((1,), dtype=torch.float32, device="cuda:0")
    st = mxq.lib().mxq_fp8_calibrate(mxq._dev_ptr(xd, "x"), m, k, ld, mxq._dev_ptr(amax, "amax"),
                                     mxq._stream_handle())
    assert st == mxq.OK
    torch.cuda.synchronize()
    assert _f32_bits(amax)[0] == oracle.fp8_calibration_amax([x]).view(np.uint32)


# ------------------------------------------------------------------ GEMM ----

@pytest.mark.parametrize("m,n,k,epi", [(256, 512, 512, mxq.EPI_NONE), (512, 1024, 1024, mxq.EPI_GELU_TANH),
                                       (100, 264, 384, mxq.EPI_NONE)])
def test_w4a8_gemm_on_static_activations(m, n, k, epi):
    say("w4a8 static gemm", m, n, k, epi)
    x = synth.activation_bf16(960 + m, m, k, ("student_t",))
    w = synth.weight_bf16(960 + m, n, k)
    amax = np.float32(float(np.abs(oracle.bf16_bits_to_f64(x)).max()) * 0.5)  # some codes saturate
    wc, ws = mxq.quantize_weight_mxfp4(dev_bf16(w))
    ac, asc = mxq.quantize_act_fp8_static(dev_bf16(x), _amax_dev(amax))
    y = mxq.gemm(mxq.W4A8, ac, asc, wc, ws, None, epi)
    torch.cuda.synchronize()
    oac, oas = oracle.fp8_quantize_static(x, amax)
    owc, ows = oracle.mxfp4_quantize(w)
    assert_codes_equal(host_u8(ac), oac, "static act codes")
    y_ref = oracle.qdq_matmul(oracle.W4A8, oac, oas, owc, ows, None, epi)
    assert_output_close(host_bits(y), y_ref, f"static w4a8 [{m}x{n}x{k}] epi={epi}")


# ------------------------------------------------------------- full size ----

def test_a14b_ffn_720p_static_full_size():
    """A14B FFN at 720p (x [75600 x 5120], 5120 -> 13824 -> 5120) with static FP8 activations:
    calibration on half of the tokens (so the other half can exceed it), sampled rows checked
    against the oracle at each stage, the second stage from the oracle's own hidden rows."""
    wl = synth.workload(3)
    up, dn = wl.linears[0], wl.linears[1]
    assert up.name == "ffn_up" and dn.name == "ffn_down"
    m = wl.m_video
    what = f"a14b ffn static [{m}x{up.n}x{up.k} -> {m}x{dn.n}x{dn.k}]"
    say(what)
    x = synth.activation_bf16(3, m, wl.dim, wl.outliers, tensor_id=synth.T_X_VIDEO)
    xd = dev_bf16(x)
    amax = mxq.fp8_calibrate(xd[: m // 2])
    torch.cuda.synchronize()
    amax_x = oracle.fp8_calibration_amax([x[: m // 2]])
    assert _f32_bits(amax)[0] == amax_x.view(np.uint32)
    rows = sample_rows(m, 24, 331)
    codes, scales = mxq.quantize_act_fp8_static(xd, amax)
    w_up = synth.weight_bf16_device(3, up.n, up.k, 0, 0, 0)
    wc_up = torch.empty((up.n, up.k // 2), dtype=torch.uint8, device="cuda:0")
    ws_up = torch.empty(mxq.mx_scale_shape(up.n, up.k), dtype=torch.uint8, device="cuda:0")
    mxq.quantize_weight_mxfp4(w_up, wc_up, ws_up)
    h = mxq.gemm(mxq.W4A8, codes, scales, wc_up, ws_up, None, up.epilogue)
    torch.cuda.synchronize()
    oac, oas = oracle.fp8_quantize_static(x[rows], amax_x)
    assert_codes_equal(host_u8(codes.index_select(0, torch.from_numpy(rows).cuda())), oac, what + " x codes")
    assert np.all(_f32_bits(scales) == oas[0].view(np.uint32))
    owc_up, ows_up = oracle.mxfp4_quantize(host_bits(w_up))
    del w_up
    h_ref = oracle.qdq_matmul(oracle.W4A8, oac, oas, owc_up, ows_up, None, up.epilogue)
    del owc_up, ows_up
    assert_output_close(host_bits(h.index_select(0, torch.from_numpy(rows).cuda())), h_ref, what + " up")
    # stage 2: the sampled rows take the oracle's bf16 hidden values; the static amax of h
    # comes from those rows (an oracle value), so other rows may saturate
    h_bits = oracle.f64_to_bf16_bits(h_ref)
    h.index_copy_(0, torch.from_numpy(rows).cuda(), dev_bf16(h_bits))
    amax_h = oracle.fp8_calibration_amax([h_bits])
    codes2, scales2 = mxq.quantize_act_fp8_static(h, _amax_dev(amax_h))
    w_dn = synth.weight_bf16_device(3, dn.n, dn.k, 0, 0, 1)
    wc_dn = torch.empty((dn.n, dn.k // 2), dtype=torch.uint8, device="cuda:0")
    ws_dn = torch.empty(mxq.mx_scale_shape(dn.n, dn.k), dtype=torch.uint8, device="cuda:0")
    mxq.quantize_weight_mxfp4(w_dn, wc_dn, ws_dn)
    y = mxq.gemm(mxq.W4A8, codes2, scales2, wc_dn, ws_dn, None, dn.epilogue)
    torch.cuda.synchronize()
    oac2, oas2 = oracle.fp8_quantize_static(h_bits, amax_h)
    assert_codes_equal(host_u8(codes2.index_select(0, torch.from_numpy(rows).cuda())), oac2, what + " h codes")
    cols = sample_rows(dn.n, 256, 332)
    owc_dn, ows_dn = oracle.mxfp4_quantize(host_bits(w_dn.index_select(0, torch.from_numpy(cols).cuda())))
    y_ref = oracle.qdq_matmul(oracle.W4A8, oac2, oas2, owc_dn, ows_dn, None, dn.epilogue)
    y_got = host_bits(y.index_select(0, torch.from_numpy(rows).cuda()).index_select(1, torch.from_numpy(cols).cuda()))
    rep = assert_output_close(y_got, y_ref, what + " down")
    say(f"{what}: worst/bound {rep['worst_ratio']:.3f}")


# -------------------------------------- fused W4A8 GEMM -> static FP8 -------
#
# mxq_gemm_fp8_static_out is defined as the static FP8 quantization of the bf16
# output the plain W4A8 GEMM writes: it must equal that two-step path byte for
# byte over the whole buffers, and, wherever the GPU's bf16 output equals the
# oracle's bf16 rounding of its QDQ result, the oracle's static codes.

def _fused_paths(m, n, k, seed, epilogue, bias, amax_frac):
    x = synth.activation_bf16(seed, m, k, ("student_t",))
    w = synth.weight_bf16(seed + 1, n, k)
    b = synth.f32_to_bf16_bits((np.random.default_rng(seed).standard_normal(n) * 0.1).astype(np.float32)) \
        if bias else None
    ac, asc = mxq.quantize_act(mxq.W4A8, dev_bf16(x))
    wc, ws = mxq.quantize_weight_mxfp4(dev_bf16(w))
    bd = dev_bf16(b) if bias else None
    y = mxq.gemm(mxq.W4A8, ac, asc, wc, ws, bd, epilogue)
    torch.cuda.synchronize()
    # the output's static amax: a fraction of the oracle's largest |h| over a few
    # rows (a calibration value, so some outputs may exceed it)
    owc, ows = oracle.mxfp4_quantize(w)
    oac, oas = oracle.fp8_quantize_per_token(x)
    b64 = oracle.bf16_bits_to_f64(b) if bias else None
    h_ref = oracle.f64_to_bf16_bits(oracle.qdq_matmul(mxq.W4A8, oac, oas, owc, ows, b64, epilogue))
    amax = np.float32(float(oracle.fp8_calibration_amax([h_ref])) * amax_frac)
    ad = _amax_dev(amax)
    rc, rs = mxq.quantize_act_fp8_static(y, ad)
    fc, fs = mxq.gemm_fp8_static_out(ac, asc, wc, ws, ad, bd, epilogue)
    torch.cuda.synchronize()
    return y, h_ref, amax, (rc, rs), (fc, fs)


FUSED_FP8_SHAPES = [(256, 512, 512), (300, 288, 384), (600, 1280, 896), (2250, 7424, 512)]


@pytest.mark.parametrize("m,n,k", FUSED_FP8_SHAPES)
@pytest.mark.parametrize("epilogue,bias,amax_frac", [(mxq.EPI_GELU_TANH, False, 1.0), (mxq.EPI_NONE, True, 0.25),
                                                     (mxq.EPI_GELU_TANH, True, 0.5), (mxq.EPI_NONE, False, 0.0)])
def test_fused_fp8_static_equals_gemm_then_quantize(m, n, k, epilogue, bias, amax_frac):
    say("fused fp8 vs two-step", m, n, k, epilogue, bias, amax_frac)
    assert mxq.gemm_fp8_static_out_supported(m, n, k)
    y, h_ref, amax, (rc, rs), (fc, fs) = _fused_paths(m, n, k, 41 + m + n, epilogue, bias, amax_frac)
    assert torch.equal(fs, rs), "row scales differ"
    bad = int((fc != rc).sum())
    assert bad == 0, f"{bad} code bytes differ"
    # tie to the oracle where the bf16 outputs agree
    agree = host_bits(y) == h_ref
    assert agree.mean() > 0.9, f"only {agree.mean():.3f} of the outputs agree in bf16"
    want_c, want_s = oracle.fp8_quantize_static(h_ref, amax)
    got = host_u8(fc)
    assert np.all(host_f32(fs).view(np.uint32) == want_s.view(np.uint32))
    bad = np.argwhere(agree & (got != want_c))
    assert bad.size == 0, f"{len(bad)} codes of agreeing outputs differ from the oracle, first {bad[:5].tolist()}"
    if 0 < amax_frac < 1:
        assert np.any((got & 0x7F) == 0x7E)  # saturation is exercised


def test_fused_fp8_static_tiny_scale():
    """A tiny static amax (pre-scaled divisor): every nonzero output saturates, zeros keep their sign."""
    m, n, k = 256, 512, 512
    say("fused fp8 tiny scale", m, n, k)
    x = synth.activation_bf16(97, m, k, ("student_t",))
    w = synth.weight_bf16(98, n, k)
    ac, asc = mxq.quantize_act(mxq.W4A8, dev_bf16(x))
    wc, ws = mxq.quantize_weight_mxfp4(dev_bf16(w))
    y = mxq.gemm(mxq.W4A8, ac, asc, wc, ws, None, mxq.EPI_GELU_TANH)
    ad = _amax_dev(1e-38)
    rc, rs = mxq.quantize_act_fp8_static(y, ad)
    fc, fs = mxq.gemm_fp8_static_out(ac, asc, wc, ws, ad, None, mxq.EPI_GELU_TANH)
    torch.cuda.synchronize()
    assert torch.equal(fc, rc) and torch.equal(fs, rs)
    yb = host_bits(y)
    got = host_u8(fc)
    nz = (yb & 0x7FFF) != 0
    assert np.all((got[nz] & 0x7F) == 0x7E) and np.all((got[~nz] & 0x7F) == 0)
    assert np.all((got >> 7) == (yb >> 15))  # signs, zeros included


def test_fused_fp8_static_a14b_ffn_up_full_size():
    """A14B FFN first projection at 720p (75600 x 13824 x 5120, GELU), whole buffers against the two-step path."""
    wl = synth.workload(3)
    up = wl.linears[0]
    m, n, k = wl.m_video, up.n, up.k
    say("fused fp8 full size", m, n, k)
    assert up.name == "ffn_up" and mxq.gemm_fp8_static_out_supported(m, n, k)
    g = torch.Generator(device="cuda:0").manual_seed(7)
    x = (torch.randn((m, k), generator=g, device="cuda:0") * 0.5).to(torch.bfloat16)
    ac, asc = mxq.quantize_act(mxq.W4A8, x)
    del x
    w = synth.weight_bf16_device(3, n, k, 0, 0, 0)
    wc, ws = mxq.quantize_weight_mxfp4(w)
    del w
    y = mxq.gemm(mxq.W4A8, ac, asc, wc, ws, None, up.epilogue)
    amax = mxq.fp8_calibrate(y[: m // 3])  # calibrated on a third of the tokens
    rc, rs = mxq.quantize_act_fp8_static(y, amax)
    del y
    fc, fs = mxq.gemm_fp8_static_out(ac, asc, wc, ws, amax, None, up.epilogue)
    torch.cuda.synchronize()
    assert torch.equal(fc, rc) and torch.equal(fs, rs)
