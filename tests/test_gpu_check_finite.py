"""The optional non-finite guard (MXQ_CHECK_FINITE): with it set, a bf16 input
holding an infinity or NaN is refused with MXQ_ERR_NONFINITE before anything
is written, and a GEMM whose bf16 output overflows reports it; with it unset,
the same calls run (non-finite inputs give unspecified results)."""

import contextlib
import ctypes
import os
import sys

import numpy as np
import pytest
import torch

import mx_bit_quantized_amd as mxq
import synth
from gpu_util import dev_bf16

pytestmark = pytest.mark.gpu

INF, NAN, BIG = 0x7F80, 0x7FC1, 0x7F7F  # bf16 +inf, a NaN, the largest finite value


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@contextlib.contextmanager
def guard(on):
    old = os.environ.get("MXQ_CHECK_FINITE")
    os.environ["MXQ_CHECK_FINITE"] = "1" if on else "0"
    try:
        yield
    finally:
        if old is None:
            os.environ.pop("MXQ_CHECK_FINITE", None)
        else:
            os.environ["MXQ_CHECK_FINITE"] = old


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _quantize(mode, x_bits):
    m, k = x_bits.shape
    codes, scales = mxq.act_buffers(mode, m, k, "cuda:0")
    codes.fill_(0x5A)
    scales.fill_(0x5A) if mode == mxq.W4A4 else scales.fill_(3.0)
    st = mxq.lib().mxq_quantize_act(int(mode), _ptr(dev_bf16(x_bits)), m, k, k, _ptr(codes), _ptr(scales),
                                     mxq._stream_handle())
    torch.cuda.synchronize()
    untouched = bool(torch.all(codes == 0x5A)) and (bool(torch.all(scales == 0x5A)) if mode == mxq.W4A4
                                                     else bool(torch.all(scales == 3.0)))
    return st, untouched


@pytest.mark.parametrize("mode", [mxq.W4A4, mxq.W4A8])
@pytest.mark.parametrize("bad", [INF, INF | 0x8000, NAN])
@pytest.mark.parametrize("where", [(0, 0), (130, 517), (255, 1023)])
def test_nonfinite_activation_is_refused(mode, bad, where):
    say("nonfinite act", mode, hex(bad), where)
    x = synth.activation_bf16(3, 256, 1024, ("student_t",))
    x[where] = bad
    with guard(True):
        st, untouched = _quantize(mode, x)
    assert st == mxq.ERR_NONFINITE and untouched
    with guard(False):
        st, _ = _quantize(mode, x)
    assert st == mxq.OK
    x[where] = BIG
    with guard(True):
        st, untouched = _quantize(mode, x)
    assert st == mxq.OK and not untouched


def test_nonfinite_weight_is_refused():
    say("nonfinite weight")
    w = synth.weight_bf16(4, 300, 512)
    w[299, 511] = INF
    codes = torch.full((300, 256), 0x5A, dtype=torch.uint8, device="cuda:0")
    scales = torch.full(mxq.mx_scale_shape(300, 512), 0x5A, dtype=torch.uint8, device="cuda:0")
    with guard(True):
        st = mxq.lib().mxq_quantize_weight_mxfp4(_ptr(dev_bf16(w)), 300, 512, 512, _ptr(codes), _ptr(scales),
                                                  mxq._stream_handle())
    torch.cuda.synchronize()
    assert st == mxq.ERR_NONFINITE and bool(torch.all(codes == 0x5A)) and bool(torch.all(scales == 0x5A))


@pytest.mark.parametrize("mode", [mxq.W4A4, mxq.W4A8])
@pytest.mark.parametrize("n", [512, 100])
def test_gemm_output_overflow_is_reported(mode, n):
    """Activations of bf16's largest value times unit weights overflow bf16 in the sum."""
    say("gemm overflow", mode, n)
    m, k = 256, 512
    x = np.full((m, k), BIG, np.uint16)
    x[: m // 2] = synth.activation_bf16(5, m // 2, k, ("student_t",))  # the first half stays finite
    w = synth.f32_to_bf16_bits(np.ones((n, k), np.float32))
    wc, ws = mxq.quantize_weight_mxfp4(dev_bf16(w))
    policy = mxq.Policy([[mode]])
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")
    with guard(True):
        ac, asc = mxq.quantize_act(mode, dev_bf16(x))  # finite input: accepted
        st = mxq.lib().mxq_gemm(int(mode), _ptr(ac), _ptr(asc), _ptr(wc), _ptr(ws), None, 0, _ptr(y), m, n, k,
                                mxq._stream_handle())
        assert st == mxq.ERR_NONFINITE
        with pytest.raises(mxq.MxqError) as err:
            mxq.qlinear(policy, 0, 0, dev_bf16(x), wc, ws, y=y)
        assert err.value.status == mxq.ERR_NONFINITE
        # the finite half alone passes the guard
        yh = mxq.qlinear(policy, 0, 0, dev_bf16(x[: m // 2]), wc, ws)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(yh.float()).all())
    with guard(False):
        st = mxq.lib().mxq_gemm(int(mode), _ptr(ac), _ptr(asc), _ptr(wc), _ptr(ws), None, 0, _ptr(y), m, n, k,
                                mxq._stream_handle())
    assert st == mxq.OK
    policy.close()
