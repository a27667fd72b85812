"""GPU tests of the fused W4A4 GEMM -> transformed MXFP4 entry point
(mxq_gemm_mxfp4_hadamard_out): the FFN first projection of a transform_on
block, whose hidden state is rotated and rescaled for the second projection
inside the GEMM's epilogue.

Its result is defined as mxq_quantize_mxfp4_hadamard(mult) of the bf16 output
the plain GEMM writes. Two checks tie it to that definition and to the oracle:

* against the library's own two-step path on the same inputs, byte for byte,
  over the whole code and scale buffers (same bf16 values, the same fp32
  butterflies, factor and rounding: any difference is a defect of the fused
  epilogue);
* against the oracle directly: the oracle's float64 QDQ result, GELU and bf16
  rounding give h_ref, and the oracle's transformed quantizer gives its codes
  and scales. The rotation mixes the 128 columns of a code panel, so wherever
  the GPU's bf16 GEMM output equals h_ref on a whole 128-column panel row, the
  fused codes and scales of that panel row must equal the oracle's.

The channel factors come from the oracle's SmoothQuant rule on synthetic
maxima (host side), spread over several binades, with some channels at the
factor of a zero maximum.
"""

import sys

import numpy as np
import pytest
import torch

import mx_bit_quantized_amd as mxq
import oracle
import synth
from gpu_util import code_rows, dev_bf16, host_bits, host_u8, w4a4_waves

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


def _act_mult(seed, n):
    g = np.random.default_rng(seed)
    ax = np.ldexp(g.uniform(1, 2, n), g.integers(-6, 6, n)).astype(np.float32)
    aw = np.ldexp(g.uniform(1, 2, n), g.integers(-10, -2, n)).astype(np.float32)
    ax[::13] = 0
    act_mult, _ = oracle.smoothquant_factors(ax, aw)
    return np.asarray(act_mult, np.float32)


def _f32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda:0")


def _operands(m, n, k, seed, bias, zero_rows=False):
    x = synth.activation_bf16(seed, m, k, ("student_t",))
    if zero_rows:
        x[0] = 0          # all-zero output rows: every transform value an exact zero
        x[m // 2] = 0
    w = synth.weight_bf16(seed + 1, n, k)
    b = synth.f32_to_bf16_bits((np.random.default_rng(seed).standard_normal(n) * 0.1).astype(np.float32)) \
        if bias else None
    return x, w, b


def _both_paths(m, n, k, seed, epilogue, bias, zero_rows=False):
    x, w, b = _operands(m, n, k, seed, bias, zero_rows)
    mult = _act_mult(seed + 2, n)
    md = _f32_dev(mult)
    ac, asc = mxq.quantize_act(mxq.W4A4, dev_bf16(x))
    wc, ws = mxq.quantize_weight_mxfp4(dev_bf16(w))
    bd = dev_bf16(b) if bias else None
    y = mxq.gemm(mxq.W4A4, ac, asc, wc, ws, bd, epilogue)
    rc, rs = mxq.quantize_mxfp4_hadamard(y, md)
    fc, fs = mxq.gemm_mxfp4_hadamard_out(ac, asc, wc, ws, md, bd, epilogue)
    torch.cuda.synchronize()
    return (x, w, b, mult), y, (rc, rs), (fc, fs)


# N = 640: the last 256-column tile is half outside N; 300 / 2250 rows: a
# ragged last row tile; 2250 x 7424 and 4352 x 4096: more tiles than CUs;
# K = 512: the fewest stages the pipelined kernel takes (4).
SHAPES = [(256, 512, 512), (300, 640, 640), (600, 1280, 896), (2250, 7424, 512), (4352, 4096, 640)]


@pytest.mark.parametrize("m,n,k", SHAPES)
@pytest.mark.parametrize("epilogue,bias", [(mxq.EPI_GELU_TANH, False), (mxq.EPI_NONE, False),
                                           (mxq.EPI_GELU_TANH, True), (mxq.EPI_NONE, True)])
def test_fused_transform_equals_gemm_then_transformed_quantizer(m, n, k, epilogue, bias):
    say("fused transform vs two-step", m, n, k, epilogue, bias)
    _, _, (rc, rs), (fc, fs) = _both_paths(m, n, k, 41 + m + n, epilogue, bias, zero_rows=True)
    assert fc.shape == rc.shape and fs.shape == rs.shape
    bad_c = int((fc != rc).sum())
    bad_s = int((fs != rs).sum())
    assert bad_c == 0 and bad_s == 0, f"{bad_c} code bytes and {bad_s} scale bytes differ"


def test_fused_transform_ignores_the_wave_setting():
    """The transformed output always runs the four-wave kernel; MXQ_W4A4_WAVES=8 changes nothing."""
    m, n, k = 600, 1280, 896
    say("fused transform, eight-wave setting", m, n, k)
    with w4a4_waves(8):
        _, _, (rc, rs), (fc, fs) = _both_paths(m, n, k, 5, mxq.EPI_GELU_TANH, True)
    assert torch.equal(fc, rc) and torch.equal(fs, rs)


@pytest.mark.parametrize("m,n,k,epilogue,bias", [(300, 640, 640, mxq.EPI_GELU_TANH, False),
                                                 (600, 1280, 896, mxq.EPI_GELU_TANH, True),
                                                 (256, 512, 512, mxq.EPI_NONE, False)])
def test_fused_transform_matches_oracle_where_bf16_agrees(m, n, k, epilogue, bias):
    say("fused transform vs oracle", m, n, k, epilogue, bias)
    (x, w, b, mult), y, _, (fc, fs) = _both_paths(m, n, k, 97 + m, epilogue, bias, zero_rows=True)
    oac, oas = oracle.quantize_act(mxq.W4A4, x)
    owc, ows = oracle.mxfp4_quantize(w)
    b64 = oracle.bf16_bits_to_f64(b) if bias else None
    h_ref = oracle.f64_to_bf16_bits(oracle.qdq_matmul(mxq.W4A4, oac, oas, owc, ows, b64, epilogue))
    want_c, want_s = oracle.mxfp4_quantize_hadamard(h_ref, mult)
    got_c = code_rows(fc, m, n, 4)                                    # [m, n/2]
    got_s = host_u8(fs).transpose(1, 0, 2).reshape(m, -1)[:, : n // 32]  # [m, n/32]
    panels = n // 128
    agree = (host_bits(y) == h_ref).reshape(m, panels, 128).all(axis=2)  # panel rows with equal bf16 inputs
    assert agree.mean() > 0.5, f"only {agree.mean():.3f} of the panel rows agree in bf16"
    codes_ok = (got_c.reshape(m, panels, 64) == want_c.reshape(m, panels, 64)).all(axis=2)
    scales_ok = (got_s.reshape(m, panels, 4) == want_s.reshape(m, panels, 4)).all(axis=2)
    bad = np.argwhere(agree & ~(codes_ok & scales_ok))
    assert bad.size == 0, f"{len(bad)} panel rows with equal bf16 inputs differ from the oracle, first {bad[:5].tolist()}"


def test_fused_transform_a14b_ffn_up_full_size():
    """A14B FFN first projection at 720p (75600 x 13824 x 5120, GELU) with the transform, whole buffers."""
    wl = synth.workload(5)
    up = next(l for l in wl.linears if l.name == "ffn_up")
    m, n, k = wl.m_video, up.n, up.k
    say("fused transform full size", m, n, k)
    assert up.epilogue == mxq.EPI_GELU_TANH and mxq.gemm_mxfp4_out_supported(m, n, k)
    g = torch.Generator(device="cuda:0").manual_seed(7)
    x = (torch.randn((m, k), generator=g, device="cuda:0") * 0.5).to(torch.bfloat16)
    ac, asc = mxq.quantize_act(mxq.W4A4, x)
    del x
    w = synth.weight_bf16_device(7, n, k, 0, 0, 8)
    wc, ws = mxq.quantize_weight_mxfp4(w)
    del w
    md = _f32_dev(_act_mult(7, n))
    y = mxq.gemm(mxq.W4A4, ac, asc, wc, ws, None, up.epilogue)
    rc, rs = mxq.quantize_mxfp4_hadamard(y, md)
    del y
    fc, fs = mxq.gemm_mxfp4_hadamard_out(ac, asc, wc, ws, md, None, up.epilogue)
    torch.cuda.synchronize()
    assert torch.equal(fc, rc) and torch.equal(fs, rs)
