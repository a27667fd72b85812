"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (quantize_act then gemm on whole [M, K] activations; in a
W4A4 block the FFN's first projection writes the second one's MXFP4 input
itself, as the benchmark runs it).

Coverage per full-size linear:

* weight codes and scales of every weight row, byte for byte against the
  oracle (after undoing the library's K-panel-major code layout and
  group-major scales);
* activation codes and scales of every token row of every synthetic input
  (the oracle runs on row chunks in parallel threads; each chunk is an
  ordinary call of the oracle's quantizer);
* y on 256 sampled token rows x all N output columns, within
  |y - y_ref| <= 2^-7 |y_ref| + 1e-3 rms(y_ref) of the oracle's float64 QDQ
  result. The sample always holds the first and last row and rows of the last
  256-row tile.

The FFN pair runs stage by stage: the first projection (with GELU) is checked
on the sampled rows; then those rows of the hidden state take the oracle's
values (its bf16 rounding of h, or in the fused W4A4 path the oracle's MXFP4
codes of that rounding), and the second projection runs on the whole buffer.
Its sampled rows then have an input fixed by the oracle alone, so the second
stage is held to the same exact-code bar as the first. The fused W4A4 path is
also compared with the library's own GEMM + quantizer over the whole hidden
state, and with the oracle's codes on every 32-element block of the sampled
rows whose bf16 values the GPU and the oracle round alike.

Config 5 (2 experts x 40 blocks) is checked on all ten linears of two W4A4
and two W4A8 blocks of each expert, chosen by a seeded draw.
"""

import functools
import sys

import numpy as np
import pytest
import torch

import mx_bit_quantized_amd as mxq
import oracle
import oracle_par
import synth
from gpu_util import (assert_codes_equal, assert_output_close, code_rows, group_major_scales, host_bits, host_f32,
                      host_u8, panel_index, sample_rows)

pytestmark = pytest.mark.gpu

N_SAMPLE = 256  # token rows per GEMM check, all output columns


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    mxq.lib()
    yield
    _host_activation.cache_clear()
    _oracle_act.cache_clear()
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


@functools.lru_cache(maxsize=4)
def _oracle_act(config_id, role, mode):
    """The oracle's activation codes and scales of every row of a synthetic input."""
    x = _host_activation(config_id, role)
    return oracle_par.map_rows(lambda c: oracle.quantize_act(mode, c), x, chunk=2048)


def _to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def _idx(a):
    return torch.from_numpy(np.asarray(a, np.int64)).to("cuda:0")


def _all_code_rows(codes, rows, k):
    """Host row-major [rows, K/2] view of a whole K-panel-major MXFP4 code buffer (K % 128 == 0)."""
    assert k % 128 == 0
    return np.ascontiguousarray(host_u8(codes).reshape(k // 128, rows, 64).transpose(1, 0, 2).reshape(rows, k // 2))


def _all_scale_rows(scales, rows, k):
    """Host [rows, K/32] of whole group-major [K/128][rows][4] scales."""
    s = host_u8(scales)
    return np.ascontiguousarray(s.transpose(1, 0, 2).reshape(rows, -1)[:, : k // 32])


def _scales_rows(scales_gm, rows, kb):
    """Group-major [K/128][rows][4] device scales -> host [len(rows), K/32] for the given rows."""
    s = host_u8(scales_gm.index_select(1, _idx(rows)))
    return np.ascontiguousarray(s.transpose(1, 0, 2).reshape(len(rows), -1)[:, :kb])


def _check_act_all(mode, codes, scales, m, k, o_codes, o_scales, what):
    """Every row's activation codes and scales against the oracle's."""
    if mode == mxq.W4A4:
        assert_codes_equal(_all_code_rows(codes, m, k), o_codes, f"{what} act codes (all {m} rows)")
        assert_codes_equal(_all_scale_rows(scales, m, k), o_scales, f"{what} act scales (all rows)")
    else:
        assert_codes_equal(host_u8(codes).reshape(m, k), o_codes, f"{what} fp8 act codes (all {m} rows)")
        assert_codes_equal(host_f32(scales).view(np.uint32), np.asarray(o_scales, np.float32).view(np.uint32),
                           f"{what} fp8 act scales (all rows)")


def _check_act_rows(mode, codes, scales, m, k, rows, o_codes, o_scales, what):
    if mode == mxq.W4A4:
        assert_codes_equal(code_rows(codes, m, k, 4, rows), o_codes, f"{what} act codes")
        assert_codes_equal(_scales_rows(scales, rows, k // 32), o_scales, f"{what} act scales")
    else:
        assert_codes_equal(host_u8(codes.view(m, k).index_select(0, _idx(rows))), o_codes, f"{what} fp8 act codes")
        got = host_f32(scales.index_select(0, _idx(rows))).view(np.uint32)
        assert_codes_equal(got, np.asarray(o_scales, np.float32).view(np.uint32), f"{what} fp8 act scales")


def _pack_weight(wl, lin, li, expert, block, what):
    """Draw, pack and check every row of one weight; returns (device codes, scales, oracle codes, scales)."""
    w = synth.weight_bf16_device(wl.config_id, lin.n, lin.k, expert, block, li)
    wc = torch.empty((lin.n, lin.k // 2), dtype=torch.uint8, device="cuda:0")
    ws = torch.empty(mxq.mx_scale_shape(lin.n, lin.k), dtype=torch.uint8, device="cuda:0")
    mxq.quantize_weight_mxfp4(w, wc, ws)
    w_host = host_bits(w)
    del w
    owc, ows = oracle_par.map_rows(oracle.mxfp4_quantize, w_host, chunk=512)
    del w_host
    assert_codes_equal(_all_code_rows(wc, lin.n, lin.k), owc, f"{what} weight codes (all {lin.n} rows)")
    assert_codes_equal(_all_scale_rows(ws, lin.n, lin.k), ows, f"{what} weight scales (all rows)")
    return wc, ws, owc, ows


def _check_y(mode, y, m, n, rows, oac, oas, owc, ows, epilogue, what):
    """y on the sampled rows x all n columns; returns the oracle's float64 rows."""
    y_ref = oracle_par.map_cols(lambda c, s: oracle.qdq_matmul(mode, oac, oas, c, s, None, epilogue), owc, ows,
                                chunk=512)
    y_got = host_bits(y.view(m, n).index_select(0, _idx(rows)))
    rep = assert_output_close(y_got, y_ref, what)
    say(f"{what}: worst/bound {rep['worst_ratio']:.3f} over {y_ref.size} outputs")
    return y_ref


def _lin_index(wl, name):
    return next(i for i, l in enumerate(wl.linears) if l.name == name)


def _single_linear(wl, e, b, li, mode, codes, scales, oac, oas, seed):
    """One non-FFN linear on already quantized (and checked) activations."""
    lin = wl.linears[li]
    m = wl.m_of(lin)
    what = f"config{wl.config_id} e{e} b{b} {lin.name} mode={mode} [{m}x{lin.n}x{lin.k}]"
    assert mxq.gemm_kernel_name(mode, m, lin.n, lin.k).startswith("pipe_"), what
    wc, ws, owc, ows = _pack_weight(wl, lin, li, e, b, what)
    y = mxq.gemm(mode, codes, scales, wc, ws, None, lin.epilogue)
    torch.cuda.synchronize()
    rows = sample_rows(m, N_SAMPLE, seed)
    _check_y(mode, y, m, lin.n, rows, oac[rows], oas[rows], owc, ows, lin.epilogue, what)


def _quantized_input(wl, role, mode, what):
    """Quantize a synthetic input on the GPU and check every row against the oracle."""
    x = _host_activation(wl.config_id, role)
    m, k = x.shape
    codes, scales = mxq.quantize_act(mode, _to_dev(x))
    torch.cuda.synchronize()
    oac, oas = _oracle_act(wl.config_id, role, mode)
    _check_act_all(mode, codes, scales, m, k, oac, oas, f"{what} {role}")
    return codes, scales, oac, oas


def _ffn(wl, e, b, mode, codes, scales, oac, oas, seed, fused):
    """The FFN pair, stage-wise (see the module docstring)."""
    i_up, i_dn = _lin_index(wl, "ffn_up"), _lin_index(wl, "ffn_down")
    up, dn = wl.linears[i_up], wl.linears[i_dn]
    m = wl.m_video
    what = f"config{wl.config_id} e{e} b{b} ffn mode={mode} [{m}x{up.n}x{up.k} -> {m}x{dn.n}x{dn.k}]"
    say(what)
    assert up.epilogue == mxq.EPI_GELU_TANH and dn.k == up.n
    assert mxq.gemm_kernel_name(mode, m, up.n, up.k).startswith("pipe_")
    assert mxq.gemm_kernel_name(mode, m, dn.n, dn.k).startswith("pipe_")
    rows = sample_rows(m, N_SAMPLE, seed)

    # stage 1: GEMM + GELU -> h (bf16), checked on the sampled rows
    wc_up, ws_up, owc_up, ows_up = _pack_weight(wl, up, i_up, e, b, what + " up")
    h = mxq.gemm(mode, codes, scales, wc_up, ws_up, None, up.epilogue)
    torch.cuda.synchronize()
    h_ref = _check_y(mode, h, m, up.n, rows, oac[rows], oas[rows], owc_up, ows_up, up.epilogue, what + " up")
    del owc_up, ows_up
    h_bits = oracle.f64_to_bf16_bits(h_ref)  # the oracle's bf16 hidden rows
    ohc, ohs = oracle.quantize_act(mode, h_bits)

    if fused:
        # the benchmark's W4A4 path: the first projection writes h's MXFP4 codes
        assert mode == mxq.W4A4 and mxq.gemm_mxfp4_out_supported(m, up.n, up.k)
        hc, hs = mxq.gemm_mxfp4_out(codes, scales, wc_up, ws_up, None, up.epilogue)
        qc, qs = mxq.quantize_act(mxq.W4A4, h)
        torch.cuda.synchronize()
        assert torch.equal(hc, qc) and torch.equal(hs, qs), f"{what}: fused codes differ from GEMM + quantizer"
        del qc, qs
        # sampled rows: the oracle's codes wherever the GPU's bf16 h is the oracle's rounding
        agree = (host_bits(h.index_select(0, _idx(rows))) == h_bits).reshape(len(rows), -1, 32).all(axis=2)
        assert agree.mean() > 0.5, f"{what}: only {agree.mean():.2%} of h blocks round alike"
        got_c = code_rows(hc, m, up.n, 4, rows).reshape(len(rows), -1, 16)
        got_s = _scales_rows(hs, rows, up.n // 32)
        assert np.array_equal(got_c[agree], ohc.reshape(len(rows), -1, 16)[agree]), f"{what}: fused codes"
        assert np.array_equal(got_s[agree], ohs[agree]), f"{what}: fused scales"
        say(f"{what}: fused codes equal the oracle's on {agree.mean():.1%} of the sampled blocks")
        # stage 2 input: the sampled rows take the oracle's codes
        flat = hc.view(-1)
        flat[_idx(panel_index(m, up.n, 4, rows).reshape(-1))] = torch.from_numpy(ohc.reshape(-1)).to("cuda:0")
        hs.index_copy_(1, _idx(rows), torch.from_numpy(group_major_scales(ohs)).to("cuda:0"))
    else:
        h.index_copy_(0, _idx(rows), _to_dev(h_bits))
        hc, hs = mxq.quantize_act(mode, h)
        torch.cuda.synchronize()
        _check_act_rows(mode, hc, hs, m, up.n, rows, ohc, ohs, what + " down")
    del h

    # stage 2: the second projection on the whole hidden state
    wc_dn, ws_dn, owc_dn, ows_dn = _pack_weight(wl, dn, i_dn, e, b, what + " down")
    y = mxq.gemm(mode, hc, hs, wc_dn, ws_dn, None, dn.epilogue)
    torch.cuda.synchronize()
    _check_y(mode, y, m, dn.n, rows, ohc, ohs, owc_dn, ows_dn, dn.epilogue, what + " down")


# config 2: A14B self-attention QKV projection at 480p, W4A4
def test_config2_qkv_w4a4_full_size():
    wl = synth.workload(2)
    say("config2 qkv")
    codes, scales, oac, oas = _quantized_input(wl, "video", mxq.W4A4, "config2")
    _single_linear(wl, 0, 0, 0, mxq.W4A4, codes, scales, oac, oas, 201)


# config 3: A14B FFN at 720p, W4A8, both projections
def test_config3_ffn_w4a8_full_size():
    wl = synth.workload(3)
    say("config3 ffn")
    codes, scales, oac, oas = _quantized_input(wl, "video", mxq.W4A8, "config3")
    _ffn(wl, 0, 0, mxq.W4A8, codes, scales, oac, oas, 301, fused=False)


def _first_block_of_mode(wl, mode):
    table = wl.policy()
    for b in range(table.shape[1]):
        if int(table[0, b]) == mode:
            return b
    pytest.skip(f"{wl.name} has no block in mode {mode}")


# config 4: TI2V-5B block, mixed policy: one block of each mode
@pytest.mark.parametrize("mode", [mxq.W4A4, mxq.W4A8])
@pytest.mark.parametrize("name", ["self_q", "cross_k"])
def test_config4_attention_linears_full_size(mode, name):
    wl = synth.workload(4)
    b = _first_block_of_mode(wl, mode)
    li = _lin_index(wl, name)
    say("config4", name, mode)
    codes, scales, oac, oas = _quantized_input(wl, wl.linears[li].m_role, mode, "config4")
    _single_linear(wl, 0, b, li, mode, codes, scales, oac, oas, 400 + 10 * mode + (name == "cross_k"))


@pytest.mark.parametrize("mode", [mxq.W4A4, mxq.W4A8])
def test_config4_ffn_full_size(mode):
    wl = synth.workload(4)
    b = _first_block_of_mode(wl, mode)
    codes, scales, oac, oas = _quantized_input(wl, "video", mode, "config4")
    _ffn(wl, 0, b, mode, codes, scales, oac, oas, 420 + mode, fused=mode == mxq.W4A4)


# config 5: A14B 40-block, 2-expert stack at 720p, mixed policy. Two blocks of
# each mode per expert, drawn with a seed; all ten linears of each, in the
# benchmark's order (q, k, v share one quantization of the video input, cross
# k and v one of the text input).
def _config5_blocks(expert, mode):
    table = synth.workload(5).policy()
    cand = [b for b in range(table.shape[1]) if int(table[expert, b]) == mode]
    g = np.random.default_rng([5, expert, mode, 99])
    return sorted(int(b) for b in g.choice(cand, size=2, replace=False))


@pytest.mark.parametrize("expert", [0, 1])
@pytest.mark.parametrize("mode", [mxq.W4A4, mxq.W4A8])
@pytest.mark.parametrize("pick", [0, 1])
def test_config5_block_full_size(expert, mode, pick):
    wl = synth.workload(5)
    b = _config5_blocks(expert, mode)[pick]
    assert int(wl.policy()[expert, b]) == mode
    policy = mxq.Policy(wl.policy())
    assert policy.mode(expert, b) == mode
    policy.close()
    say(f"config5 expert {expert} block {b} mode={mode}")
    quantized = {}
    for li, lin in enumerate(wl.linears):
        if lin.m_role == "ffn_hidden":
            continue
        if lin.m_role not in quantized:
            quantized[lin.m_role] = _quantized_input(wl, lin.m_role, mode, f"config5 e{expert} b{b}")
        codes, scales, oac, oas = quantized[lin.m_role]
        if lin.name == "ffn_up":
            _ffn(wl, expert, b, mode, codes, scales, oac, oas, 5000 + 100 * expert + b, fused=mode == mxq.W4A4)
        else:
            _single_linear(wl, expert, b, li, mode, codes, scales, oac, oas, 5000 + 100 * expert + b + li)


def test_config5_blocks_span_both_experts_and_modes():
    """The seeded draw gives distinct blocks, and different ones for the two experts' W4A8 masks."""
    table = synth.workload(5).policy()
    for e in range(2):
        for mode in (mxq.W4A4, mxq.W4A8):
            bl = _config5_blocks(e, mode)
            assert len(set(bl)) == 2 and all(int(table[e, b]) == mode for b in bl)
    assert not np.array_equal(table[0], table[1])


# The pipelined kernel addresses a bf16 output per 256-row tile, with 32-bit
# offsets from the tile's first row, so the output may pass 2^31 bytes.
# M = 131071 puts the last 256-row tile one row short of full and the output
# 16 KiB under 2^31 bytes; M = 131072 gives exactly 2^31 bytes, the size at
# which offsets from the start of the output would have reached the flag bit
# the kernel uses for dropped stores. The sampled rows include the last tile.
@pytest.mark.parametrize("mode", [mxq.W4A4, mxq.W4A8])
@pytest.mark.parametrize("m,kernel", [(131071, "pipe_"), (131072, "pipe_")])
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
    oac, oas = oracle_par.map_rows(lambda c: oracle.quantize_act(mode, c), host_bits(x), chunk=4096)
    _check_act_all(mode, codes, scales, m, k, oac, oas, what)
    owc, ows = oracle.mxfp4_quantize(w)
    rows = sample_rows(m, N_SAMPLE, 70 + mode)
    _check_y(mode, y, m, n, rows, oac[rows], oas[rows], owc, ows, mxq.EPI_NONE, what)
