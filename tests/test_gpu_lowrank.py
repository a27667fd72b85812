"""GPU parity of SVDQuant's low-rank branch (mxq_lowrank_down / mxq_lowrank_up)
and of the whole SVDQuant layer built from them, against the CPU oracle.

The branch contracts in fp32 on the matrix cores; the oracle sums exactly. On
inputs whose sums are exact in fp32 the two agree bit for bit; otherwise the
bf16 results are held to |y - y_ref| <= 2^-7 |y_ref| + 1e-3 rms(y_ref).
"""

import sys

import numpy as np
import pytest
import torch

import mx_bit_quantized_amd as mxq
import oracle
import synth
from gpu_util import assert_output_close, code_rows, dev_bf16, host_bits, host_u8, sample_rows

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


def _bits(a):
    return synth.f32_to_bf16_bits(np.asarray(a, np.float32))


def _idx(a):
    return torch.from_numpy(np.asarray(a, np.int64)).to("cuda:0")


@pytest.mark.parametrize("m,k,r", [(1, 128, 32), (37, 256, 64), (300, 5120, 128), (1000, 384, 96), (4097, 128, 32),
                                   (65, 13824, 32)])
def test_lowrank_down_vs_oracle(m, k, r):
    say("lowrank down", m, k, r)
    g = np.random.default_rng(m + k + r)
    x = synth.activation_bf16(700 + m, m, k, ("student_t",))
    l1t = _bits(g.standard_normal((r, k)) * 0.05)
    t = mxq.lowrank_down(dev_bf16(x), dev_bf16(l1t))
    torch.cuda.synchronize()
    want = oracle.lowrank_down(x, l1t)
    assert_output_close(host_bits(t), oracle.bf16_bits_to_f64(want), f"T [{m}x{k}] r={r}")
    # exact sums: small integers and +-1 / 0 factors
    xi = _bits(g.integers(-4, 5, (m, k)))
    li = _bits(g.integers(-1, 2, (r, k)))
    ti = mxq.lowrank_down(dev_bf16(xi), dev_bf16(li))
    torch.cuda.synchronize()
    wi = oracle.lowrank_down(xi, li)
    exact = np.abs(oracle.bf16_bits_to_f64(wi)) <= 256  # integers up to 256 are exact in bf16
    assert np.array_equal(host_bits(ti)[exact], wi[exact])


@pytest.mark.parametrize("m,n,r,epi,inplace", [(64, 128, 32, 0, False), (300, 288, 64, 1, False),
                                               (1000, 640, 128, 1, True), (33, 96, 96, 0, True)])
def test_lowrank_up_vs_oracle(m, n, r, epi, inplace):
    say("lowrank up", m, n, r, epi, inplace)
    g = np.random.default_rng(m * n + r)
    y_pre = _bits(g.standard_normal((m, n)))
    t = _bits(g.standard_normal((m, r)))
    l2 = _bits(g.standard_normal((n, r)) * 0.1)
    yd = dev_bf16(y_pre)
    y = mxq.lowrank_up(yd, dev_bf16(t), dev_bf16(l2), epi, y=yd if inplace else None)
    torch.cuda.synchronize()
    want = oracle.lowrank_up(y_pre, t, l2, epi)
    assert_output_close(host_bits(y), oracle.bf16_bits_to_f64(want), f"y [{m}x{n}] r={r} epi={epi}")
    if epi == 0:  # exact integers
        yp = _bits(g.integers(-8, 9, (m, n)))
        ti = _bits(g.integers(-2, 3, (m, r)))
        li = _bits(g.integers(-1, 2, (n, r)))
        yi = mxq.lowrank_up(dev_bf16(yp), dev_bf16(ti), dev_bf16(li))
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(yi), oracle.lowrank_up(yp, ti, li))


def _svd_factors(w_bits, r):
    """Rank-r factors of W by an SVD (float64), split as sqrt of the singular values, in bf16,
    and the bf16 residual R = W - L2 L1^T."""
    w = oracle.bf16_bits_to_f64(w_bits)
    u, s, vt = np.linalg.svd(w, full_matrices=False)
    l2 = u[:, :r] * np.sqrt(s[:r])[None, :]          # [N, r]
    l1t = vt[:r] * np.sqrt(s[:r])[:, None]           # [r, K]
    l2b, l1tb = _bits(l2), _bits(l1t)
    res = w - oracle.bf16_bits_to_f64(l2b) @ oracle.bf16_bits_to_f64(l1tb)
    return l1tb, l2b, oracle.f64_to_bf16_bits(res)


def _lowrank_weight(n, k, seed):
    """A weight with a strong low-rank part (outlier directions) on top of N(0, 0.02) noise."""
    g = np.random.default_rng(seed)
    w = g.standard_normal((n, k)) * 0.02 + (g.standard_normal((n, 8)) @ g.standard_normal((8, k))) * 0.05
    return _bits(w)


@pytest.mark.parametrize("m,n,k,r,epi", [(256, 512, 512, 32, 0), (300, 288, 384, 64, 1), (100, 256, 256, 32, 1)])
def test_svdquant_layer_vs_oracle(m, n, k, r, epi):
    say("svdquant layer", m, n, k, r, epi)
    x = synth.activation_bf16(800 + m, m, k, ("student_t",))
    w = _lowrank_weight(n, k, 900 + n)
    l1t, l2, res = _svd_factors(w, r)
    rc, rs = mxq.quantize_weight_mxfp4(dev_bf16(res))
    xd = dev_bf16(x)
    ac, asc = mxq.quantize_act(mxq.W4A4, xd)
    y_pre = mxq.gemm(mxq.W4A4, ac, asc, rc, rs, None, mxq.EPI_NONE)
    t = mxq.lowrank_down(xd, dev_bf16(l1t))
    y = mxq.lowrank_up(y_pre, t, dev_bf16(l2), epi, y=y_pre)
    torch.cuda.synchronize()
    orc, ors = oracle.mxfp4_quantize(res)
    oac, oas = oracle.mxfp4_quantize(x)
    y_ref, _, _ = oracle.svdquant_linear(oracle.W4A4, oac, oas, orc, ors, x, l1t, l2, None, epi)
    assert_output_close(host_bits(y), oracle.bf16_bits_to_f64(y_ref), f"svdquant [{m}x{n}x{k}] r={r}")
    if epi == 0:
        # the branch's reason: against the exact bf16 product, SVDQuant beats plain W4A4 on such weights
        exact = oracle.bf16_bits_to_f64(x) @ oracle.bf16_bits_to_f64(w).T
        owc, ows = oracle.mxfp4_quantize(w)
        y_plain = oracle.qdq_matmul(oracle.W4A4, oac, oas, owc, ows)
        sq = lambda v: 10 * np.log10((exact ** 2).sum() / ((v - exact) ** 2).sum())
        assert sq(oracle.bf16_bits_to_f64(host_bits(y))) > sq(y_plain) + 1.0


def test_svdquant_a14b_ffn_up_full_size():
    """A14B FFN first projection at 720p (75600 x 13824 x 5120, GELU) with a rank-32 branch; sampled
    token rows and output columns against the oracle."""
    wl = synth.workload(5)
    up = next(l for l in wl.linears if l.name == "ffn_up")
    m, n, k, r = wl.m_video, up.n, up.k, 32
    what = f"svdquant a14b ffn up [{m}x{n}x{k}] r={r}"
    say(what)
    g = np.random.default_rng(55)
    x = synth.activation_bf16(5, m, k, wl.outliers, tensor_id=synth.T_X_VIDEO)
    res = synth.weight_bf16(5, n, k, 0, 0, 8)
    l1t = _bits(g.standard_normal((r, k)) * 0.02)
    l2 = _bits(g.standard_normal((n, r)) * 0.02)
    xd = dev_bf16(x)
    rc, rs = mxq.quantize_weight_mxfp4(dev_bf16(res))
    ac, asc = mxq.quantize_act(mxq.W4A4, xd)
    y = mxq.gemm(mxq.W4A4, ac, asc, rc, rs, None, mxq.EPI_NONE)
    t = mxq.lowrank_down(xd, dev_bf16(l1t))
    mxq.lowrank_up(y, t, dev_bf16(l2), up.epilogue, y=y)
    torch.cuda.synchronize()
    rows = sample_rows(m, 16, 61)
    cols = sample_rows(n, 256, 62)
    orc, ors = oracle.mxfp4_quantize(res[cols])
    oac, oas = oracle.mxfp4_quantize(x[rows])
    y_ref, _, _ = oracle.svdquant_linear(oracle.W4A4, oac, oas, orc, ors, x[rows], l1t, l2[cols], None, up.epilogue)
    y_got = host_bits(y.index_select(0, _idx(rows)).index_select(1, _idx(cols)))
    rep = assert_output_close(y_got, oracle.bf16_bits_to_f64(y_ref), what)
    say(f"{what}: worst/bound {rep['worst_ratio']:.3f}")


# ---- the branch inside the W4A4 GEMM (mxq_gemm_lowrank) ----------------------
# N = 640 / 1288: last 256-column tile partly outside N (1288 is no multiple of
# 128 or 256); M = 300 / 513 / 2250: ragged last row tile; 2250 x 7424: more
# tiles than CUs; K = 512: the fewest code stages the W4A4 ring takes (4).
FUSED_LR_CASES = [(256, 256, 512, 32, 0, False), (300, 640, 640, 64, 1, True), (600, 1288, 896, 96, 1, False),
                  (513, 512, 512, 128, 0, True), (2250, 7424, 512, 32, 1, False)]


def _fused_operands(m, n, k, r, seed, bias):
    g = np.random.default_rng(seed)
    x = synth.activation_bf16(seed, m, k, ("student_t",))
    res = synth.weight_bf16(seed + 1, n, k)
    l1t = _bits(g.standard_normal((r, k)) * 0.02)
    l2 = _bits(g.standard_normal((n, r)) * 0.05)
    b = _bits(g.standard_normal(n) * 0.1) if bias else None
    return x, res, l1t, l2, b


def _fused_gpu(x, res, l1t, l2, b, epi, mxfp4_out=False):
    xd = dev_bf16(x)
    rc, rs = mxq.quantize_weight_mxfp4(dev_bf16(res))
    ac, asc = mxq.quantize_act(mxq.W4A4, xd)
    t = mxq.lowrank_down(xd, dev_bf16(l1t))
    bd = dev_bf16(b) if b is not None else None
    y = mxq.gemm_lowrank(ac, asc, rc, rs, t, dev_bf16(l2), bd, epi, mxfp4_out=mxfp4_out)
    torch.cuda.synchronize()
    return y


def _fused_oracle(x, res, l1t, l2, b, epi):
    orc, ors = oracle.mxfp4_quantize(res)
    oac, oas = oracle.mxfp4_quantize(x)
    t = oracle.lowrank_down(x, l1t)
    b64 = oracle.bf16_bits_to_f64(b) if b is not None else None
    return oracle.svdquant_linear_fused(oracle.W4A4, oac, oas, orc, ors, t, l2, b64, epi)


@pytest.mark.parametrize("m,n,k,r,epi,bias", FUSED_LR_CASES)
def test_gemm_lowrank_vs_oracle(m, n, k, r, epi, bias):
    what = f"gemm+branch [{m}x{n}x{k}] r={r} epi={epi} bias={bias}"
    say(what)
    assert mxq.gemm_lowrank_supported(m, n, k)
    ops = _fused_operands(m, n, k, r, 1000 + m + n + r, bias)
    y = _fused_gpu(*ops, epi)
    rep = assert_output_close(host_bits(y), _fused_oracle(*ops, epi), what)
    say(f"{what}: worst/bound {rep['worst_ratio']:.3f}")


@pytest.mark.parametrize("m,n,k,r", [(256, 512, 512, 64), (300, 264, 640, 32), (520, 1032, 512, 128)])
def test_gemm_lowrank_exact_sums(m, n, k, r):
    """Operands whose every sum is exact in fp32 (MXFP4-exact activations and residual, small
    integer branch factors): the GPU's bf16 output equals the oracle's rounding bit for bit, so a
    misplaced branch element, rank panel or row shows up as a wrong bit."""
    say("gemm+branch exact", m, n, k, r)
    g = np.random.default_rng(m + n + r)
    x = _bits(g.choice([-2.0, -1.0, -0.5, 0.0, 0.5, 1.0, 2.0, 3.0], (m, k)))
    res = _bits(g.choice([-1.5, -0.5, 0.0, 0.5, 1.0, 2.0], (n, k)))
    l1t = _bits(g.integers(-1, 2, (r, k)) * (g.random((r, k)) < 0.05))
    l2 = _bits(g.integers(-2, 3, (n, r)))
    b = _bits(g.integers(-8, 9, n))
    for epi in (mxq.EPI_NONE,):
        y = _fused_gpu(x, res, l1t, l2, b, epi)
        want = oracle.f64_to_bf16_bits(_fused_oracle(x, res, l1t, l2, b, epi))
        got = host_bits(y)
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"{len(bad)} outputs differ, first {bad[:5].tolist()}"


@pytest.mark.parametrize("m,n,k,r,epi,bias", [(300, 640, 640, 64, 1, True), (2250, 7424, 512, 32, 1, False),
                                              (256, 512, 512, 128, 0, False)])
def test_gemm_lowrank_mxfp4_out(m, n, k, r, epi, bias):
    """MXFP4 output: byte for byte the library's quantizer applied to the bf16 output of the same
    call, and the oracle's codes wherever the bf16 values agree with the oracle's on a whole block."""
    say("gemm+branch -> mxfp4", m, n, k, r, epi, bias)
    ops = _fused_operands(m, n, k, r, 2000 + m + r, bias)
    y = _fused_gpu(*ops, epi)
    fc, fs = _fused_gpu(*ops, epi, mxfp4_out=True)
    rc, rs = mxq.quantize_act(mxq.W4A4, y)
    torch.cuda.synchronize()
    assert torch.equal(fc, rc) and torch.equal(fs, rs)
    h_ref = oracle.f64_to_bf16_bits(_fused_oracle(*ops, epi))
    want_c, want_s = oracle.quantize_act(mxq.W4A4, h_ref)
    got_c = code_rows(fc, m, n, 4)
    got_s = host_u8(fs).transpose(1, 0, 2).reshape(m, -1)[:, : n // 32]
    agree = (host_bits(y) == h_ref).reshape(m, n // 32, 32).all(axis=2)
    assert agree.mean() > 0.9, f"only {agree.mean():.3f} of the blocks agree in bf16"
    ok = (got_c.reshape(m, n // 32, 16) == want_c.reshape(m, n // 32, 16)).all(axis=2) & (got_s == want_s)
    bad = np.argwhere(agree & ~ok)
    assert bad.size == 0, f"{len(bad)} blocks differ from the oracle, first {bad[:5].tolist()}"


def test_gemm_lowrank_a14b_ffn_up_full_size():
    """A14B FFN first projection at 720p (75600 x 13824 x 5120, GELU) with the rank-32 branch in
    the GEMM: sampled rows and columns against the oracle; the MXFP4 output against the library's
    quantizer on the bf16 output, whole buffers."""
    wl = synth.workload(5)
    up = next(l for l in wl.linears if l.name == "ffn_up")
    m, n, k, r = wl.m_video, up.n, up.k, 32
    what = f"gemm+branch a14b ffn up [{m}x{n}x{k}] r={r}"
    say(what)
    g = np.random.default_rng(56)
    x = synth.activation_bf16(5, m, k, wl.outliers, tensor_id=synth.T_X_VIDEO)
    res = synth.weight_bf16(5, n, k, 0, 0, 8)
    l1t = _bits(g.standard_normal((r, k)) * 0.02)
    l2 = _bits(g.standard_normal((n, r)) * 0.02)
    xd = dev_bf16(x)
    rc, rs = mxq.quantize_weight_mxfp4(dev_bf16(res))
    ac, asc = mxq.quantize_act(mxq.W4A4, xd)
    t = mxq.lowrank_down(xd, dev_bf16(l1t))
    del xd
    l2d = dev_bf16(l2)
    y = mxq.gemm_lowrank(ac, asc, rc, rs, t, l2d, None, up.epilogue)
    torch.cuda.synchronize()
    rows = sample_rows(m, 16, 63)
    cols = sample_rows(n, 256, 64)
    y_got = host_bits(y.index_select(0, _idx(rows)).index_select(1, _idx(cols)))
    y_ref = _fused_oracle(x[rows], res[cols], l1t, l2[cols], None, up.epilogue)
    rep = assert_output_close(y_got, y_ref, what)
    say(f"{what}: worst/bound {rep['worst_ratio']:.3f}")
    qc, qs = mxq.quantize_act(mxq.W4A4, y)
    del y
    fc, fs = mxq.gemm_lowrank(ac, asc, rc, rs, t, l2d, None, up.epilogue, mxfp4_out=True)
    torch.cuda.synchronize()
    assert torch.equal(fc, qc) and torch.equal(fs, qs)


# ---- the activation quantizer fused with the branch's first half -------------
@pytest.mark.parametrize("m,k,r", [(1, 128, 32), (37, 256, 64), (300, 5120, 128), (1000, 384, 96), (4097, 640, 32),
                                   (65, 13824, 32)])
def test_quantize_act_lowrank_matches_both_calls_and_oracle(m, k, r):
    """Codes and scales byte for byte those of the W4A4 quantizer and of the oracle's MXFP4 rule;
    t bit for bit that of the down kernel alone, and within the tolerance of the oracle."""
    say("quantize+down", m, k, r)
    g = np.random.default_rng(3 * m + k + r)
    x = synth.activation_bf16(900 + m, m, k, ("student_t",))
    l1t = _bits(g.standard_normal((r, k)) * 0.05)
    xd, ld = dev_bf16(x), dev_bf16(l1t)
    qc, qs, t = mxq.quantize_act_lowrank(xd, ld)
    rc, rs = mxq.quantize_act(mxq.W4A4, xd)
    t_alone = mxq.lowrank_down(xd, ld)
    torch.cuda.synchronize()
    assert torch.equal(qc, rc) and torch.equal(qs, rs)
    assert torch.equal(t, t_alone)
    want_c, want_s = oracle.mxfp4_quantize(x)
    assert np.array_equal(code_rows(qc, m, k, 4), want_c)
    assert np.array_equal(host_u8(qs).transpose(1, 0, 2).reshape(m, -1)[:, : k // 32], want_s)
    assert_output_close(host_bits(t), oracle.bf16_bits_to_f64(oracle.lowrank_down(x, l1t)), f"t [{m}x{k}] r={r}")


def test_quantize_act_lowrank_edge_blocks():
    """Zero rows, blocks at the largest bf16 exponents and subnormal-only blocks: the fused
    quantizer takes the same scale bytes and codes as the oracle."""
    say("quantize+down edge blocks")
    m, k = 70, 256
    g = np.random.default_rng(4)
    x = synth.activation_bf16(44, m, k, ("student_t",)).copy()
    x[0] = 0
    x[1, :32] = 0x7F7F                      # bf16 max in a whole block
    x[2, 32:64] = 0x0001                    # smallest subnormal
    x[3, 64:96] = (g.integers(1, 0x7F, 32) | 0x8000).astype(np.uint16)  # negative subnormals
    x[69, 96:128] = 0x8000                  # negative zeros
    l1t = _bits(g.standard_normal((32, k)) * 0.05)
    qc, qs, _ = mxq.quantize_act_lowrank(dev_bf16(x), dev_bf16(l1t))
    torch.cuda.synchronize()
    want_c, want_s = oracle.mxfp4_quantize(x)
    assert np.array_equal(code_rows(qc, m, k, 4), want_c)
    assert np.array_equal(host_u8(qs).transpose(1, 0, 2).reshape(m, -1)[:, : k // 32], want_s)


def test_quantize_act_lowrank_a14b_full_size():
    """The A14B video activation at 720p (75600 x 5120) with a rank-32 branch, as the bench runs it:
    whole code and scale buffers against the quantizer, t against the down kernel, sampled rows of
    both against the oracle."""
    wl = synth.workload(5)
    m, k, r = wl.m_video, wl.dim, 32
    what = f"quantize+down a14b [{m}x{k}] r={r}"
    say(what)
    g = np.random.default_rng(57)
    x = synth.activation_bf16(5, m, k, wl.outliers, tensor_id=synth.T_X_VIDEO)
    l1t = _bits(g.standard_normal((r, k)) * 0.02)
    xd, ld = dev_bf16(x), dev_bf16(l1t)
    qc, qs, t = mxq.quantize_act_lowrank(xd, ld)
    rc, rs = mxq.quantize_act(mxq.W4A4, xd)
    t_alone = mxq.lowrank_down(xd, ld)
    torch.cuda.synchronize()
    assert torch.equal(qc, rc) and torch.equal(qs, rs)
    assert torch.equal(t, t_alone)
    rows = sample_rows(m, 24, 65)
    want_c, want_s = oracle.mxfp4_quantize(x[rows])
    assert np.array_equal(code_rows(qc, m, k, 4, rows), want_c)
    got_s = host_u8(qs).transpose(1, 0, 2)[rows].reshape(len(rows), -1)
    assert np.array_equal(got_s, want_s)
    rep = assert_output_close(host_bits(t.index_select(0, _idx(rows))),
                              oracle.bf16_bits_to_f64(oracle.lowrank_down(x[rows], l1t)), what)
    say(f"{what}: worst/bound {rep['worst_ratio']:.3f}")
