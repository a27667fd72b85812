"""GPU tests of the fused W4A4 GEMM -> MXFP4 entry point (mxq_gemm_mxfp4_out).

Its result is defined as the MXFP4 quantization of the bf16 output the plain
GEMM writes. Two checks tie it to that definition and to the oracle:

* against the library's own two-step path on the same inputs, byte for byte,
  over the whole code and scale buffers (same bf16 values, same rule: any
  difference is a defect of the fused epilogue);
* against the oracle directly: the oracle's float64 QDQ result, GELU and bf16
  rounding give h_ref, and the oracle's MXFP4 quantizer gives its codes and
  scales. Wherever the GPU's bf16 GEMM output equals h_ref on a whole 32-wide
  block (the plain GEMM's own oracle tests bound it everywhere), the fused
  codes and scale of that block must equal the oracle's.
"""

import sys

import numpy as np
import pytest
import torch

import mx_bit_quantized_amd as mxq
import oracle
import synth
from gpu_util import W4A4_WAVE_KERNEL, code_rows, dev_bf16, host_bits, host_u8, w4a4_waves

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


def _operands(m, n, k, seed, bias):
    x = synth.activation_bf16(seed, m, k, ("student_t",))
    w = synth.weight_bf16(seed + 1, n, k)
    b = synth.f32_to_bf16_bits((np.random.default_rng(seed).standard_normal(n) * 0.1).astype(np.float32)) \
        if bias else None
    return x, w, b


def _both_paths(m, n, k, seed, epilogue, bias):
    x, w, b = _operands(m, n, k, seed, bias)
    ac, asc = mxq.quantize_act(mxq.W4A4, dev_bf16(x))
    wc, ws = mxq.quantize_weight_mxfp4(dev_bf16(w))
    bd = dev_bf16(b) if bias else None
    y = mxq.gemm(mxq.W4A4, ac, asc, wc, ws, bd, epilogue)
    rc, rs = mxq.quantize_act(mxq.W4A4, y)
    fc, fs = mxq.gemm_mxfp4_out(ac, asc, wc, ws, bd, epilogue)
    torch.cuda.synchronize()
    return (x, w, b), (ac, asc, wc, ws), y, (rc, rs), (fc, fs)


# N = 640: the last 256-column tile is half outside N; 300 / 2250 rows: a
# ragged last row tile; 2250 x 7424 and 4352 x 4096: more tiles than CUs.
FUSED_SHAPES = [(256, 512, 512), (300, 640, 640), (600, 1280, 896), (2250, 7424, 512), (4352, 4096, 640)]


@pytest.mark.parametrize("waves", [4, 8])
@pytest.mark.parametrize("m,n,k", FUSED_SHAPES)
@pytest.mark.parametrize("epilogue,bias", [(mxq.EPI_GELU_TANH, False), (mxq.EPI_NONE, False),
                                           (mxq.EPI_GELU_TANH, True), (mxq.EPI_NONE, True)])
def test_fused_equals_gemm_then_quantize(waves, m, n, k, epilogue, bias):
    say("fused vs two-step", waves, m, n, k, epilogue, bias)
    with w4a4_waves(waves):
        assert mxq.gemm_kernel_name(mxq.W4A4, m, n, k) == W4A4_WAVE_KERNEL[waves]
        _, _, _, (rc, rs), (fc, fs) = _both_paths(m, n, k, 31 + m + n, epilogue, bias)
    assert fc.shape == rc.shape and fs.shape == rs.shape
    bad_c = int((fc != rc).sum())
    bad_s = int((fs != rs).sum())
    assert bad_c == 0 and bad_s == 0, f"{bad_c} code bytes and {bad_s} scale bytes differ"


@pytest.mark.parametrize("waves", [4, 8])
@pytest.mark.parametrize("m,n,k,epilogue,bias", [(300, 640, 640, mxq.EPI_GELU_TANH, False),
                                                 (600, 1280, 896, mxq.EPI_GELU_TANH, True),
                                                 (256, 512, 512, mxq.EPI_NONE, False)])
def test_fused_matches_oracle_where_bf16_agrees(waves, m, n, k, epilogue, bias):
    say("fused vs oracle", waves, m, n, k, epilogue, bias)
    with w4a4_waves(waves):
        assert mxq.gemm_kernel_name(mxq.W4A4, m, n, k) == W4A4_WAVE_KERNEL[waves]
        (x, w, b), _, y, _, (fc, fs) = _both_paths(m, n, k, 77 + m, epilogue, bias)
    oac, oas = oracle.quantize_act(mxq.W4A4, x)
    owc, ows = oracle.mxfp4_quantize(w)
    b64 = oracle.bf16_bits_to_f64(b) if bias else None
    h_ref = oracle.f64_to_bf16_bits(oracle.qdq_matmul(mxq.W4A4, oac, oas, owc, ows, b64, epilogue))
    want_c, want_s = oracle.quantize_act(mxq.W4A4, h_ref)
    got_c = code_rows(fc, m, n, 4)                                    # [m, n/2]
    got_s = host_u8(fs).transpose(1, 0, 2).reshape(m, -1)[:, : n // 32]  # [m, n/32]
    agree = (host_bits(y) == h_ref).reshape(m, n // 32, 32).all(axis=2)  # blocks with equal bf16 inputs
    assert agree.mean() > 0.9, f"only {agree.mean():.3f} of the blocks agree in bf16"
    blk_codes_ok = (got_c.reshape(m, n // 32, 16) == want_c.reshape(m, n // 32, 16)).all(axis=2)
    bad = np.argwhere(agree & ~(blk_codes_ok & (got_s == want_s)))
    assert bad.size == 0, f"{len(bad)} blocks with equal bf16 inputs differ from the oracle, first {bad[:5].tolist()}"


def test_fused_a14b_ffn_up_full_size():
    """A14B FFN first projection at 720p (75600 x 13824 x 5120, GELU), whole buffers."""
    wl = synth.workload(5)
    up = next(l for l in wl.linears if l.name == "ffn_up")
    m, n, k = wl.m_video, up.n, up.k
    say("fused full size", m, n, k)
    assert up.epilogue == mxq.EPI_GELU_TANH and mxq.gemm_kernel_name(mxq.W4A4, m, n, k).startswith("pipe_")
    g = torch.Generator(device="cuda:0").manual_seed(5)
    x = (torch.randn((m, k), generator=g, device="cuda:0") * 0.5).to(torch.bfloat16)
    ac, asc = mxq.quantize_act(mxq.W4A4, x)
    del x
    w = synth.weight_bf16_device(5, n, k, 0, 0, 8)
    wc, ws = mxq.quantize_weight_mxfp4(w)
    del w
    y = mxq.gemm(mxq.W4A4, ac, asc, wc, ws, None, up.epilogue)
    rc, rs = mxq.quantize_act(mxq.W4A4, y)
    del y
    fc, fs = mxq.gemm_mxfp4_out(ac, asc, wc, ws, None, up.epilogue)
    torch.cuda.synchronize()
    assert torch.equal(fc, rc) and torch.equal(fs, rs)
