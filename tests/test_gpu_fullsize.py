"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (quantize_act then gemm on whole [M, K] activations).

The oracle cannot run a whole 75600-token linear in seconds, so each case is
checked on a sample of outputs it can compute one by one. Both quantizers act
row by row (an MXFP4 block lies inside one row along K; the FP8 scale belongs
to one token), so:

* weight codes and scales of sampled weight rows must match the oracle byte
  for byte (every row of the FFN's first projection, which the second stage
  needs whole), after undoing the library's K-panel-major code layout;
* activation codes and scales of sampled token rows likewise;
* y on the grid (sampled token rows) x (sampled output columns) must satisfy
  |y - y_ref| <= 2^-7 |y_ref| + 1e-3 rms(y_ref) against the oracle's float64
  QDQ result.

Samples always hold the first and last row and column and the last 256-wide
tile, so ragged tails and the far corner of the grid are covered.

The FFN pair runs stage by stage: the first projection (with GELU) is checked
on the sampled rows, then the oracle's bf16 rounding of those rows is written
into the hidden buffer, and the second projection quantizes and multiplies the
whole buffer. Its sampled rows then have an input fixed by the oracle alone,
so the second stage is held to the same exact-code bar as the first.
"""

import functools
import sys

import numpy as np
import pytest
import torch

import mx_bit_quantized_amd as mxq
import oracle
import synth
from gpu_util import assert_codes_equal, assert_output_close, code_rows, host_bits, host_f32, host_u8, sample_rows

pytestmark = pytest.mark.gpu

N_ROWS = 24    # random token rows per case (plus edges)
N_COLS = 256   # random output columns per case (plus edges)


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    mxq.lib()
    yield
    _host_activation.cache_clear()
    torch.cuda.synchronize()


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=2)
def _host_activation(config_id, role):
    wl = synth.workload(config_id)
    m = wl.m_text if role == "text" else wl.m_video
    tid = synth.T_X_TEXT if role == "text" else synth.T_X_VIDEO
    return synth.activation_bf16(config_id, m, wl.dim, wl.outliers, tensor_id=tid)


def _to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def _idx(a):
    return torch.from_numpy(np.asarray(a, np.int64)).to("cuda:0")


def _scales_rows(scales_gm, rows, kb):
    """Group-major [K/128][rows][4] device scales -> host [len(rows), K/32] for the given rows."""
    s = host_u8(scales_gm.index_select(1, _idx(rows)))
    return np.ascontiguousarray(s.transpose(1, 0, 2).reshape(len(rows), -1)[:, :kb])


def _check_act(mode, codes, scales, rows, o_codes, o_scales, what):
    if mode == mxq.W4A4:  # K-panel-major byte buffer [rows, K/2]
        got = code_rows(codes, codes.shape[0], codes.shape[1] * 2, 4, rows)
    else:  # row-major FP8 codes
        got = host_u8(codes.index_select(0, _idx(rows)))
    assert_codes_equal(got, o_codes, f"{what} act codes")
    if mode == mxq.W4A4:
        assert_codes_equal(_scales_rows(scales, rows, o_scales.shape[1]), o_scales, f"{what} act scales")
    else:
        got = host_f32(scales.index_select(0, _idx(rows))).view(np.uint32)
        assert_codes_equal(got, np.asarray(o_scales, np.float32).view(np.uint32), f"{what} act fp8 scales")


def _check_weight_rows(w_dev, wc, ws, rows, k, what):
    """Oracle-pack the sampled weight rows and compare with the device pack; returns the oracle's."""
    w_rows = host_bits(w_dev.index_select(0, _idx(rows)))
    owc, ows = oracle.mxfp4_quantize(w_rows)
    assert_codes_equal(code_rows(wc, wc.shape[0], k, 4, rows), owc, f"{what} weight codes")
    assert_codes_equal(_scales_rows(ws, rows, k // 32), ows, f"{what} weight scales")
    return owc, ows


def _pack_weight(wl, lin, li, expert, block):
    w = synth.weight_bf16_device(wl.config_id, lin.n, lin.k, expert, block, li)
    wc = torch.empty((lin.n, lin.k // 2), dtype=torch.uint8, device="cuda:0")
    ws = torch.empty(mxq.mx_scale_shape(lin.n, lin.k), dtype=torch.uint8, device="cuda:0")
    mxq.quantize_weight_mxfp4(w, wc, ws)
    return w, wc, ws


def _block_of_mode(wl, mode):
    table = wl.policy()
    for e in range(table.shape[0]):
        for b in range(table.shape[1]):
            if int(table[e, b]) == mode:
                return e, b
    pytest.skip(f"{wl.name} has no block in mode {mode}")


def _lin_index(wl, name):
    return next(i for i, l in enumerate(wl.linears) if l.name == name)


def _single_linear_case(config_id, mode, name, seed):
    wl = synth.workload(config_id)
    e, b = _block_of_mode(wl, mode)
    li = _lin_index(wl, name)
    lin = wl.linears[li]
    m = wl.m_of(lin)
    what = f"config{config_id} e{e} b{b} {name} mode={mode} [{m}x{lin.n}x{lin.k}]"
    say(what)
    policy = mxq.Policy(wl.policy())
    assert policy.mode(e, b) == mode
    policy.close()
    assert mxq.gemm_kernel_name(mode, m, lin.n, lin.k).startswith("pipe_")
    x = _host_activation(config_id, lin.m_role)
    w, wc, ws = _pack_weight(wl, lin, li, e, b)
    codes, scales = mxq.quantize_act(mode, _to_dev(x))
    y = mxq.gemm(mode, codes, scales, wc, ws, None, lin.epilogue)
    torch.cuda.synchronize()
    rows = sample_rows(m, N_ROWS, seed)
    cols = sample_rows(lin.n, N_COLS, seed + 1)
    owc, ows = _check_weight_rows(w, wc, ws, cols, lin.k, what)
    oac, oas = oracle.quantize_act(mode, x[rows])
    _check_act(mode, codes, scales, rows, oac, oas, what)
    y_ref = oracle.qdq_matmul(mode, oac, oas, owc, ows, None, lin.epilogue)
    y_got = host_bits(y.index_select(0, _idx(rows)).index_select(1, _idx(cols)))
    rep = assert_output_close(y_got, y_ref, what)
    say(f"{what}: worst/bound {rep['worst_ratio']:.3f}")


def _ffn_case(config_id, mode, seed):
    wl = synth.workload(config_id)
    e, b = _block_of_mode(wl, mode)
    i_up, i_dn = _lin_index(wl, "ffn_up"), _lin_index(wl, "ffn_down")
    up, dn = wl.linears[i_up], wl.linears[i_dn]
    m = wl.m_video
    what = f"config{config_id} e{e} b{b} ffn mode={mode} [{m}x{up.n}x{up.k} -> {m}x{dn.n}x{dn.k}]"
    say(what)
    assert up.epilogue == mxq.EPI_GELU_TANH and dn.k == up.n
    assert mxq.gemm_kernel_name(mode, m, up.n, up.k).startswith("pipe_")
    assert mxq.gemm_kernel_name(mode, m, dn.n, dn.k).startswith("pipe_")
    x = _host_activation(config_id, "video")
    rows = sample_rows(m, N_ROWS, seed)

    # stage 1: x -> quantize -> GEMM + GELU -> h (bf16)
    w_up, wc_up, ws_up = _pack_weight(wl, up, i_up, e, b)
    codes, scales = mxq.quantize_act(mode, _to_dev(x))
    h = mxq.gemm(mode, codes, scales, wc_up, ws_up, None, up.epilogue)
    torch.cuda.synchronize()
    owc_up, ows_up = _check_weight_rows(w_up, wc_up, ws_up, np.arange(up.n), up.k, what + " up")
    del w_up
    oac, oas = oracle.quantize_act(mode, x[rows])
    _check_act(mode, codes, scales, rows, oac, oas, what + " up")
    del codes, scales
    h_ref = oracle.qdq_matmul(mode, oac, oas, owc_up, ows_up, None, up.epilogue)
    del owc_up, ows_up
    rep = assert_output_close(host_bits(h.index_select(0, _idx(rows))), h_ref, what + " up")
    say(f"{what} up: worst/bound {rep['worst_ratio']:.3f}")

    # stage 2: the sampled rows of h take the oracle's bf16 values, then h -> quantize -> GEMM -> y
    h_bits = oracle.f64_to_bf16_bits(h_ref)
    h.index_copy_(0, _idx(rows), _to_dev(h_bits))
    w_dn, wc_dn, ws_dn = _pack_weight(wl, dn, i_dn, e, b)
    codes, scales = mxq.quantize_act(mode, h)
    y = mxq.gemm(mode, codes, scales, wc_dn, ws_dn, None, dn.epilogue)
    torch.cuda.synchronize()
    cols = sample_rows(dn.n, N_COLS, seed + 1)
    owc_dn, ows_dn = _check_weight_rows(w_dn, wc_dn, ws_dn, cols, dn.k, what + " down")
    oac2, oas2 = oracle.quantize_act(mode, h_bits)
    _check_act(mode, codes, scales, rows, oac2, oas2, what + " down")
    y_ref = oracle.qdq_matmul(mode, oac2, oas2, owc_dn, ows_dn, None, dn.epilogue)
    y_got = host_bits(y.index_select(0, _idx(rows)).index_select(1, _idx(cols)))
    rep = assert_output_close(y_got, y_ref, what + " down")
    say(f"{what} down: worst/bound {rep['worst_ratio']:.3f}")


# config 2: A14B self-attention QKV projection at 480p, W4A4
def test_config2_qkv_w4a4_full_size():
    _single_linear_case(2, mxq.W4A4, "qkv", 201)


# config 3: A14B FFN at 720p, W4A8, both projections
def test_config3_ffn_w4a8_full_size():
    _ffn_case(3, mxq.W4A8, 301)


# config 4: TI2V-5B block, mixed policy: one block of each mode
@pytest.mark.parametrize("mode", [mxq.W4A4, mxq.W4A8])
@pytest.mark.parametrize("name", ["self_q", "cross_k"])
def test_config4_attention_linears_full_size(mode, name):
    _single_linear_case(4, mode, name, 400 + 10 * mode + (name == "cross_k"))


@pytest.mark.parametrize("mode", [mxq.W4A4, mxq.W4A8])
def test_config4_ffn_full_size(mode):
    _ffn_case(4, mode, 420 + mode)


# config 5: A14B 40-block, 2-expert stack at 720p, mixed policy
@pytest.mark.parametrize("mode", [mxq.W4A4, mxq.W4A8])
@pytest.mark.parametrize("name", ["self_o", "cross_v"])
def test_config5_attention_linears_full_size(mode, name):
    _single_linear_case(5, mode, name, 500 + 10 * mode + (name == "cross_v"))


@pytest.mark.parametrize("mode", [mxq.W4A4, mxq.W4A8])
def test_config5_ffn_full_size(mode):
    _ffn_case(5, mode, 520 + mode)


# The pipelined kernel addresses its output with 32-bit buffer offsets and takes
# shapes whose bf16 output stays below 2^31 - 256 bytes; one row more and the
# direct kernel (64-bit addresses) takes the shape. M = 131071 puts the last
# 256-row tile one row short of full and the output 16 KiB under the bound;
# M = 131072 gives exactly 2^31 bytes of output.
@pytest.mark.parametrize("mode", [mxq.W4A4, mxq.W4A8])
@pytest.mark.parametrize("m,kernel", [(131071, "pipe_"), (131072, "direct_")])
def test_gemm_at_the_output_size_bound(mode, m, kernel):
    n, k = 8192, 512
    what = f"output bound mode={mode} [{m}x{n}x{k}] {kernel}"
    say(what)
    assert mxq.gemm_kernel_name(mode, m, n, k).startswith(kernel)
    g = torch.Generator(device="cuda:0").manual_seed(m + mode)
    x = torch.randn((m, k), generator=g, device="cuda:0").to(torch.bfloat16)
    w = synth.weight_bf16(31, n, k)
    wc, ws = mxq.quantize_weight_mxfp4(_to_dev(w))
    codes, scales = mxq.quantize_act(mode, x)
    y = mxq.gemm(mode, codes, scales, wc, ws, None, mxq.EPI_NONE)
    torch.cuda.synchronize()
    rows = sample_rows(m, N_ROWS, 70 + mode)
    cols = sample_rows(n, N_COLS, 71 + mode)
    x_rows = host_bits(x.index_select(0, _idx(rows)))
    oac, oas = oracle.quantize_act(mode, x_rows)
    _check_act(mode, codes, scales, rows, oac, oas, what)
    owc, ows = oracle.mxfp4_quantize(w[cols])
    y_ref = oracle.qdq_matmul(mode, oac, oas, owc, ows, None, mxq.EPI_NONE)
    y_got = host_bits(y.index_select(0, _idx(rows)).index_select(1, _idx(cols)))
    rep = assert_output_close(y_got, y_ref, what)
    say(f"{what}: worst/bound {rep['worst_ratio']:.3f}")
