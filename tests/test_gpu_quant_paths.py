"""GPU parity of quantizer paths the shape tests above do not reach, called
through the C ABI directly.

* FP8 per-token rows longer than a wave's registers hold (K > 14336 takes the
  two-pass row kernel: an amax pass over the row, then the quantizing pass),
  at the boundary and past it;
* leading dimensions larger than K (ldx, ldw > K) for mxq_quantize_act in both
  modes and for mxq_quantize_weight_mxfp4: the padding columns hold huge
  values, so a kernel that read them would change the amax and every code of
  the row.

Codes and scales must equal the oracle's byte for byte (FP8 scales as fp32
bit patterns), with the MXFP4 layouts undone on the host.
"""

import sys

import numpy as np
import pytest
import torch

import mx_bit_quantized_amd as mxq
import oracle
import synth
from gpu_util import assert_codes_equal, code_rows, dev_bf16, group_major_scales, host_f32, host_u8

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


def _bit(v):
    """bf16 bit pattern of one float, as an int."""
    return int(_bits([v])[0])


def _rows_with_edges(m, k, seed):
    """Student-t outlier rows plus a zero row, a subnormal row, FP8 ties and a huge row."""
    g = np.random.default_rng(seed)
    x = synth.activation_bf16(seed, m, k, ("student_t",))
    x[1] = 0
    x[2] = (g.integers(0, 0x80, k) | (g.integers(0, 2, k) << 15)).astype(np.uint16)
    # values whose quotient by s = 448 / 448 = 1 lands on E4M3 ties (row amax 448)
    x[3] = _bits(g.choice([1.0625, 2.125, 4.25, 17.0, 208.0, -0.0], k))
    x[3, 0] = _bit(448.0)
    x[4] = _bits(g.standard_normal(k) * 1e30)
    x[5, k - 1] = _bit(-3e4)  # the row amax sits in the last element
    return x


def _padded(x, ld, fill):
    """[m, K] bf16 bits -> [m, ld] with the extra columns set to ``fill`` (bf16 bits)."""
    m, k = x.shape
    out = np.full((m, ld), fill, np.uint16)
    out[:, :k] = x
    return out


def _abi_quantize_act(mode, xp, m, k, ld):
    xd = dev_bf16(xp)
    codes, scales = mxq.act_buffers(mode, m, k, "cuda:0")
    st = mxq.lib().mxq_quantize_act(int(mode), mxq._dev_ptr(xd, "x"), m, k, ld, mxq._dev_ptr(codes, "codes"),
                                     mxq._dev_ptr(scales, "scales"), mxq._stream_handle())
    assert st == mxq.OK, mxq.status_string(st)
    torch.cuda.synchronize()
    return codes, scales


def _check_act(mode, codes, scales, x, what):
    m, k = x.shape
    want_c, want_s = oracle.quantize_act(mode, x)
    if mode == mxq.W4A4:
        assert_codes_equal(host_u8(scales), group_major_scales(want_s), f"{what} mxfp4 scales")
        assert_codes_equal(code_rows(codes, m, k, 4), want_c, f"{what} mxfp4 codes")
    else:
        assert_codes_equal(host_f32(scales).view(np.uint32), want_s.view(np.uint32), f"{what} fp8 scales")
        assert_codes_equal(host_u8(codes), want_c, f"{what} fp8 codes")


# K = 14336 is the longest row the one-pass kernel keeps in registers (28
# chunks of 8 per lane); 14368 is the first row length of the two-pass kernel.
@pytest.mark.parametrize("k", [14336, 14368, 16384, 20480])
def test_fp8_per_token_long_rows(k):
    m = 67
    say("fp8 long rows", m, k)
    x = _rows_with_edges(m, k, 600 + k % 1000)
    codes, scales = _abi_quantize_act(mxq.W4A8, x, m, k, k)
    _check_act(mxq.W4A8, codes, scales, x, f"fp8 [{m}x{k}]")


@pytest.mark.parametrize("mode", [mxq.W4A4, mxq.W4A8])
@pytest.mark.parametrize("m,k,ld", [(40, 96, 104), (37, 512, 640), (9, 5120, 5184), (33, 16384, 16392)])
def test_quantize_act_leading_dimension(mode, m, k, ld):
    say("quantize_act ld", mode, m, k, ld)
    x = _rows_with_edges(m, k, 700 + m)
    for fill in (_bit(3e38), 0x8000):
        xp = _padded(x, ld, int(fill))
        codes, scales = _abi_quantize_act(mode, xp, m, k, ld)
        _check_act(mode, codes, scales, x, f"mode={mode} [{m}x{k}] ld={ld} fill={int(fill):#06x}")


@pytest.mark.parametrize("n,k,ldw", [(40, 96, 128), (300, 160, 168), (64, 5120, 5376)])
def test_quantize_weight_leading_dimension(n, k, ldw):
    say("quantize_weight ld", n, k, ldw)
    w = synth.weight_bf16(7, n, k)
    w[0, :32] = 0
    wp = _padded(w, ldw, _bit(-2e38))
    wd = dev_bf16(wp)
    codes = torch.empty((n, k // 2), dtype=torch.uint8, device="cuda:0")
    scales = torch.empty(mxq.mx_scale_shape(n, k), dtype=torch.uint8, device="cuda:0")
    st = mxq.lib().mxq_quantize_weight_mxfp4(mxq._dev_ptr(wd, "w"), n, k, ldw, mxq._dev_ptr(codes, "codes"),
                                              mxq._dev_ptr(scales, "scales"), mxq._stream_handle())
    assert st == mxq.OK, mxq.status_string(st)
    torch.cuda.synchronize()
    want_c, want_s = oracle.mxfp4_quantize(w)
    assert_codes_equal(host_u8(scales), group_major_scales(want_s), "weight scales")
    assert_codes_equal(code_rows(codes, n, k, 4), want_c, "weight codes")
