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
from gpu_util import assert_output_close, dev_bf16, host_bits, sample_rows

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
