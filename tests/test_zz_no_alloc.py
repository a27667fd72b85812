"""The allocation-free qlinear (mxq_qlinear_noalloc) against mxq_qlinear, through the C ABI.

Both run the same kernels on the same inputs, so y must be equal bit for bit.
Two calls in a row per mode, the second with a smaller input (the scratch
area keeps the first call's codes; the second must not depend on them), then
the size limit: the largest problem the scratch holds runs, and one token row
more is refused with MXQ_ERR_SCRATCH before anything is written."""

import ctypes
import sys

import numpy as np
import pytest
import torch

import mx_bit_quantized_amd as mxq
import synth
from gpu_util import dev_bf16

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _both(policy, x, wc, ws, bias, epilogue):
    """y from mxq_qlinear (with a torch workspace) and from mxq_qlinear_noalloc."""
    L = mxq.lib()
    m, k = x.shape
    n = wc.shape[0]
    mode = policy.mode(0, 0)
    work = torch.empty((mxq.qlinear_workspace_bytes(mode, m, k),), dtype=torch.uint8, device="cuda:0")
    y_ref = torch.full((m, n), 3.0, dtype=torch.bfloat16, device="cuda:0")
    y = torch.full((m, n), -5.0, dtype=torch.bfloat16, device="cuda:0")
    S = mxq._stream_handle()
    st = L.mxq_qlinear(policy.handle, 0, 0, _ptr(x), m, k, _ptr(wc), _ptr(ws), n, _ptr(bias), epilogue, _ptr(y_ref),
                       _ptr(work), work.numel(), S)
    assert st == mxq.OK, mxq.status_string(st)
    st = L.mxq_qlinear_noalloc(policy.handle, 0, 0, _ptr(x), m, k, _ptr(wc), _ptr(ws), n, _ptr(bias), epilogue,
                               _ptr(y), S)
    assert st == mxq.OK, mxq.status_string(st)
    torch.cuda.synchronize()
    return y_ref, y


@pytest.mark.parametrize("mode", [mxq.W4A4, mxq.W4A8])
def test_noalloc_equals_qlinear_on_two_calls_second_smaller(mode):
    policy = mxq.Policy([[mode]])
    for i, (m, n, k, epi, bias) in enumerate([(4096, 1024, 5120, mxq.EPI_GELU_TANH, False),
                                               (300, 512, 1024, mxq.EPI_NONE, True)]):
        say("noalloc", mode, i, m, n, k)
        x = dev_bf16(synth.activation_bf16(70 + i, m, k, ("student_t",)))
        wc, ws = mxq.quantize_weight_mxfp4(dev_bf16(synth.weight_bf16(80 + i, n, k)))
        b = dev_bf16(synth.f32_to_bf16_bits(np.random.default_rng(i).standard_normal(n).astype(np.float32) * 0.1)) \
            if bias else None
        y_ref, y = _both(policy, x, wc, ws, b, epi)
        assert torch.equal(y, y_ref), f"mode={mode} call {i}: noalloc differs from qlinear"
    policy.close()


@pytest.mark.parametrize("mode", [mxq.W4A4, mxq.W4A8])
def test_noalloc_size_limit(mode):
    k, n = 5120, 256
    # the largest M whose workspace fits the scratch area, then one row more
    m = 1
    while mxq.qlinear_workspace_bytes(mode, 2 * m, k) <= mxq.NOALLOC_SCRATCH_BYTES:
        m *= 2
    lo, hi = m, 2 * m
    while hi - lo > 1:
        mid = (lo + hi) // 2
        lo, hi = (mid, hi) if mxq.qlinear_workspace_bytes(mode, mid, k) <= mxq.NOALLOC_SCRATCH_BYTES else (lo, mid)
    m_max = lo
    say("noalloc limit", mode, m_max)
    policy = mxq.Policy([[mode]])
    x = (torch.randn((m_max + 1, k), device="cuda:0") * 0.5).to(torch.bfloat16)
    wc, ws = mxq.quantize_weight_mxfp4(dev_bf16(synth.weight_bf16(90, n, k)))
    y_ref, y = _both(policy, x[:m_max], wc, ws, None, mxq.EPI_NONE)
    assert torch.equal(y, y_ref)
    y2 = torch.full((m_max + 1, n), 7.0, dtype=torch.bfloat16, device="cuda:0")
    st = mxq.lib().mxq_qlinear_noalloc(policy.handle, 0, 0, _ptr(x), m_max + 1, k, _ptr(wc), _ptr(ws), n, None,
                                       mxq.EPI_NONE, _ptr(y2), mxq._stream_handle())
    assert st == mxq.ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.all(y2 == 7.0)
    policy.close()
