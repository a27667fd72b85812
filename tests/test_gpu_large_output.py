"""GPU tests of row-major GEMM outputs larger than 2 GiB.

The pipelined kernel addresses a bf16 (or static FP8) output per tile of 256
rows, so the output may exceed 2^31 bytes, as a stacked q+k+v projection at
720p does (75600 x 15360 bf16, 2.3 GB). Two checks per case:

* the stacked GEMM against separate GEMMs on column slices of the weight,
  byte for byte (each output column is computed the same way whatever N is);
* sampled rows (row 0, rows past 2^31 / (2 N) where the old 32-bit offsets
  would have wrapped, and the ragged last tile) against the oracle, within the
  output tolerance.

The same column-slice check covers the GEMM with SVDQuant's branch on the
stacked shape and the stacked cross-attention k+v on the 512 text tokens.
"""

import sys

import numpy as np
import pytest
import torch

import mx_bit_quantized_amd as mxq
import oracle
import synth
from gpu_util import W4A4_WAVE_KERNEL, assert_output_close, host_bits, w4a4_waves

pytestmark = pytest.mark.gpu

M, K = 75600, 512            # 720p tokens; a short K keeps the cases quick
N_STACK, N_PART = 15360, 5120
ROWS = [0, 1, 255, 69905, 70000, 75519, 75520, 75599]   # 2^31 / (2 * 15360) = 69905.07; last tile from 75520


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    mxq.lib()
    yield
    torch.cuda.synchronize()


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def operands():
    g = torch.Generator(device="cuda:0").manual_seed(17)
    x = (torch.randn((M, K), generator=g, device="cuda:0")).to(torch.bfloat16)
    w = synth.weight_bf16(17, N_STACK, K)
    return x, w


def _x_rows(x):
    return host_bits(x[ROWS])


@pytest.mark.parametrize("mode,waves", [(mxq.W4A4, 4), (mxq.W4A4, 8), (mxq.W4A8, 4)])
def test_bf16_output_past_2gib(operands, mode, waves):
    x, w = operands
    say("bf16 output > 2 GiB", mode, waves, M, N_STACK, K)
    assert M * N_STACK * 2 > 2 ** 31
    with w4a4_waves(waves):
        assert mxq.gemm_kernel_name(mode, M, N_STACK, K) == (W4A4_WAVE_KERNEL[waves] if mode == mxq.W4A4
                                                              else "pipe_w4a8_wg256x256_wave128x128")
        wd = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).to("cuda:0")
        wc, ws = mxq.quantize_weight_mxfp4(wd)
        ac, asc = mxq.quantize_act(mode, x)
        y = mxq.gemm(mode, ac, asc, wc, ws, None, mxq.EPI_GELU_TANH)
        parts = []
        for p in range(N_STACK // N_PART):
            wpc, wps = mxq.quantize_weight_mxfp4(wd[p * N_PART:(p + 1) * N_PART])
            parts.append(mxq.gemm(mode, ac, asc, wpc, wps, None, mxq.EPI_GELU_TANH))
        torch.cuda.synchronize()
    for p, yp in enumerate(parts):
        assert torch.equal(y[:, p * N_PART:(p + 1) * N_PART], yp), f"column slice {p} differs from its own GEMM"
    del parts
    oac, oas = oracle.quantize_act(mode, _x_rows(x))
    owc, ows = oracle.mxfp4_quantize(w)
    y_ref = oracle.qdq_matmul(mode, oac, oas, owc, ows, None, mxq.EPI_GELU_TANH)
    assert_output_close(host_bits(y[ROWS]), y_ref, f"rows {ROWS} of the {M}x{N_STACK} output")


def test_static_fp8_output_past_2gib(operands):
    x, _ = operands
    n = 28672  # M * n bytes of codes = 2.17 GB
    say("static FP8 output > 2 GiB", M, n, K)
    assert M * n > 2 ** 31 and mxq.gemm_fp8_static_out_supported(M, n, K)
    w = synth.weight_bf16_device(17, n, K, 0, 0, 1)
    wc, ws = mxq.quantize_weight_mxfp4(w)
    del w
    ac, asc = mxq.quantize_act(mxq.W4A8, x)
    y = mxq.gemm(mxq.W4A8, ac, asc, wc, ws, None, mxq.EPI_GELU_TANH)
    amax = mxq.fp8_calibrate(y)
    rc, rs = mxq.quantize_act_fp8_static(y, amax)
    del y
    fc, fs = mxq.gemm_fp8_static_out(ac, asc, wc, ws, amax, None, mxq.EPI_GELU_TANH)
    torch.cuda.synchronize()
    assert torch.equal(fc, rc) and torch.equal(fs, rs)


def test_lowrank_bf16_output_past_2gib(operands):
    """The GEMM with SVDQuant's branch on the stacked shape: each output column is its slice's own
    GEMM with the branch (the same codes, T and L2 row), byte for byte, past 2 GiB of output."""
    x, w = operands
    r = 32
    say("gemm+branch bf16 output > 2 GiB", M, N_STACK, K, r)
    assert mxq.gemm_lowrank_supported(M, N_STACK, K)
    g = torch.Generator(device="cuda:0").manual_seed(23)
    t = (torch.randn((M, r), generator=g, device="cuda:0") * 0.5).to(torch.bfloat16)
    l2 = (torch.randn((N_STACK, r), generator=g, device="cuda:0") * 0.05).to(torch.bfloat16)
    wd = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    wc, ws = mxq.quantize_weight_mxfp4(wd)
    ac, asc = mxq.quantize_act(mxq.W4A4, x)
    y = mxq.gemm_lowrank(ac, asc, wc, ws, t, l2, None, mxq.EPI_GELU_TANH)
    torch.cuda.synchronize()
    for p in range(N_STACK // N_PART):
        wpc, wps = mxq.quantize_weight_mxfp4(wd[p * N_PART:(p + 1) * N_PART])
        yp = mxq.gemm_lowrank(ac, asc, wpc, wps, t, l2[p * N_PART:(p + 1) * N_PART].contiguous(), None,
                              mxq.EPI_GELU_TANH)
        torch.cuda.synchronize()
        assert torch.equal(y[:, p * N_PART:(p + 1) * N_PART], yp), f"column slice {p} differs from its own GEMM"
        del yp


@pytest.mark.parametrize("waves", [4, 8])
def test_stacked_text_projection_equals_slices(waves):
    """Cross-attention k+v on the 512 text tokens as one GEMM (512 x 10240 x 5120, the eight-wave kernel
    by default): each half equals its own GEMM byte for byte, as for the stacked video projections."""
    m, n_part, k = 512, 5120, 5120
    say("stacked text k+v", m, 2 * n_part, k, waves)
    x = synth.activation_bf16(31, m, k, ("student_t",))
    w = synth.weight_bf16(32, 2 * n_part, k)
    with w4a4_waves(waves):
        xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to("cuda:0")
        wd = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).to("cuda:0")
        ac, asc = mxq.quantize_act(mxq.W4A4, xd)
        wc, ws = mxq.quantize_weight_mxfp4(wd)
        y = mxq.gemm(mxq.W4A4, ac, asc, wc, ws, None, mxq.EPI_NONE)
        parts = []
        for p in range(2):
            wpc, wps = mxq.quantize_weight_mxfp4(wd[p * n_part:(p + 1) * n_part])
            parts.append(mxq.gemm(mxq.W4A4, ac, asc, wpc, wps, None, mxq.EPI_NONE))
        torch.cuda.synchronize()
    for p, yp in enumerate(parts):
        assert torch.equal(y[:, p * n_part:(p + 1) * n_part], yp), f"half {p} differs from its own GEMM"
    oac, oas = oracle.quantize_act(mxq.W4A4, x[:64])
    owc, ows = oracle.mxfp4_quantize(w)
    y_ref = oracle.qdq_matmul(mxq.W4A4, oac, oas, owc, ows, None, mxq.EPI_NONE)
    assert_output_close(host_bits(y[:64]), y_ref, "first 64 rows of the stacked text projection")
