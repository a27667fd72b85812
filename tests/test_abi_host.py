"""The C ABI on the host: library loads, exports what include/mxq.h declares,
and rejects bad arguments before any HIP call (no GPU needed)."""

import ctypes
import os
import re

import numpy as np
import pytest

import mx_bit_quantized_amd as mxq
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "mxq.h")
FAKE = ctypes.c_void_p(0x10000)        # 16-byte aligned, never dereferenced
FAKE_ODD = ctypes.c_void_p(0x10008)    # 8-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mxq_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = mxq.lib()
    names = declared_functions()
    assert len(names) == 31, names
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(mxq._SIGS)


def test_status_strings_and_version():
    assert mxq.version() == 10100
    for st in range(10):
        assert mxq.status_string(st)
    assert mxq.status_string(99) == "unknown status"


def test_quantize_act_rejects_modes_shapes_nulls_alignment():
    L = mxq.lib()
    S = None
    # bf16 and transform_on policy values are not quantized-linear modes
    for mode in (mxq.POLICY_BF16, mxq.POLICY_TRANSFORM_ON, -1, 7):
        assert L.mxq_quantize_act(mode, FAKE, 4, 64, 64, FAKE, FAKE, S) == mxq.ERR_MODE
    for k in (0, 16, 48, -32):
        assert L.mxq_quantize_act(mxq.W4A4, FAKE, 4, k, 64, FAKE, FAKE, S) == mxq.ERR_SHAPE
    assert L.mxq_quantize_act(mxq.W4A4, FAKE, -1, 64, 64, FAKE, FAKE, S) == mxq.ERR_SHAPE
    assert L.mxq_quantize_act(mxq.W4A4, FAKE, 4, 64, 32, FAKE, FAKE, S) == mxq.ERR_SHAPE  # ld < K
    assert L.mxq_quantize_act(mxq.W4A4, FAKE, 1 << 31, 64, 64, FAKE, FAKE, S) == mxq.ERR_SHAPE
    assert L.mxq_quantize_act(mxq.W4A8, None, 4, 64, 64, FAKE, FAKE, S) == mxq.ERR_NULL
    assert L.mxq_quantize_act(mxq.W4A8, FAKE, 4, 64, 64, None, FAKE, S) == mxq.ERR_NULL
    assert L.mxq_quantize_act(mxq.W4A8, FAKE_ODD, 4, 64, 64, FAKE, FAKE, S) == mxq.ERR_ALIGN
    assert L.mxq_quantize_act(mxq.W4A8, FAKE, 4, 64, 68, FAKE, FAKE, S) == mxq.ERR_ALIGN  # ld % 8
    # empty problems enqueue nothing and accept null pointers
    assert L.mxq_quantize_act(mxq.W4A4, None, 0, 64, 64, None, None, S) == mxq.OK


def test_mxfp4_layout_validation():
    L = mxq.lib()
    S = None
    for fn in (L.mxq_mxfp4_to_canonical, L.mxq_mxfp4_from_canonical):
        for k in (0, 16, 48, -32):
            assert fn(FAKE, FAKE, 4, k, FAKE, FAKE, S) == mxq.ERR_SHAPE
        assert fn(FAKE, FAKE, -1, 64, FAKE, FAKE, S) == mxq.ERR_SHAPE
        assert fn(FAKE, FAKE, 1 << 31, 64, FAKE, FAKE, S) == mxq.ERR_SHAPE
        for i in range(4):
            args = [FAKE] * 4
            args[i] = None
            assert fn(args[0], args[1], 4, 64, args[2], args[3], S) == mxq.ERR_NULL
            args[i] = FAKE_ODD
            assert fn(args[0], args[1], 4, 64, args[2], args[3], S) == mxq.ERR_ALIGN
        # no rows: nothing enqueued, null pointers accepted
        assert fn(None, None, 0, 64, None, None, S) == mxq.OK


def test_qlinear_noalloc_validation():
    """Checks that come before the scratch area is touched (no GPU needed)."""
    L = mxq.lib()
    assert L.mxq_qlinear_noalloc(None, 0, 0, FAKE, 4, 64, FAKE, FAKE, 64, None, 0, FAKE, None) == mxq.ERR_NULL
    for mode, m in ((mxq.W4A4, 1 << 20), (mxq.W4A8, 100000)):
        p = mxq.Policy([[mode]])
        assert mxq.qlinear_workspace_bytes(mode, m, 5120) > mxq.NOALLOC_SCRATCH_BYTES
        assert L.mxq_qlinear_noalloc(p.handle, 0, 0, FAKE, m, 5120, FAKE, FAKE, 64, None, 0, FAKE,
                                     None) == mxq.ERR_SCRATCH
        assert L.mxq_qlinear_noalloc(p.handle, 0, 1, FAKE, 4, 64, FAKE, FAKE, 64, None, 0, FAKE,
                                     None) == mxq.ERR_RANGE
        assert L.mxq_qlinear_noalloc(p.handle, 0, 0, FAKE, 4, 48, FAKE, FAKE, 64, None, 0, FAKE,
                                     None) == mxq.ERR_SHAPE
        p.close()
    p = mxq.Policy([[mxq.POLICY_TRANSFORM_ON]])
    assert L.mxq_qlinear_noalloc(p.handle, 0, 0, FAKE, 4, 128, FAKE, FAKE, 64, None, 0, FAKE, None) == mxq.ERR_MODE
    p.close()


def test_weight_pack_and_gemm_validation():
    L = mxq.lib()
    S = None
    assert L.mxq_quantize_weight_mxfp4(FAKE, 8, 40, 40, FAKE, FAKE, S) == mxq.ERR_SHAPE
    assert L.mxq_quantize_weight_mxfp4(None, 8, 64, 64, FAKE, FAKE, S) == mxq.ERR_NULL
    assert L.mxq_quantize_weight_mxfp4(FAKE, 8, 64, 64, FAKE_ODD, FAKE, S) == mxq.ERR_ALIGN
    assert L.mxq_quantize_weight_mxfp4(None, 0, 64, 64, None, None, S) == mxq.OK
    args = [FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, 4, 8, 64, S]
    assert L.mxq_gemm(2, *args) == mxq.ERR_MODE
    bad_epi = list(args)
    bad_epi[5] = 2
    assert L.mxq_gemm(mxq.W4A4, *bad_epi) == mxq.ERR_MODE
    bad_k = list(args)
    bad_k[9] = 100
    assert L.mxq_gemm(mxq.W4A4, *bad_k) == mxq.ERR_SHAPE
    bad_n = list(args)
    bad_n[8] = -3
    assert L.mxq_gemm(mxq.W4A4, *bad_n) == mxq.ERR_SHAPE
    null_y = list(args)
    null_y[6] = None
    assert L.mxq_gemm(mxq.W4A8, *null_y) == mxq.ERR_NULL
    odd_bias = list(args)
    odd_bias[4] = FAKE_ODD
    assert L.mxq_gemm(mxq.W4A8, *odd_bias) == mxq.ERR_ALIGN
    empty = list(args)
    empty[7] = 0
    empty[0] = None
    assert L.mxq_gemm(mxq.W4A8, *empty) == mxq.OK


def test_gemm_mxfp4_out_validation():
    """Host-side checks of the fused GEMM -> MXFP4 entry point (nothing is enqueued)."""
    L = mxq.lib()
    S = None
    # a0 as0 w0 ws0 bias epi yc ys M N K stream
    ok = [FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, FAKE, 512, 1024, 1024, S]
    bad_epi = list(ok)
    bad_epi[5] = 2
    assert L.mxq_gemm_mxfp4_out(*bad_epi) == mxq.ERR_MODE
    bad_k = list(ok)
    bad_k[10] = 100
    assert L.mxq_gemm_mxfp4_out(*bad_k) == mxq.ERR_SHAPE
    # shapes the pipelined kernel does not take, or N not a multiple of 128
    for m, n, k in [(255, 1024, 1024), (512, 1024, 384), (512, 1000, 1024), (512, 1088, 1024)]:
        args = list(ok)
        args[8:11] = [m, n, k]
        assert L.mxq_gemm_mxfp4_out(*args) == mxq.ERR_SHAPE, (m, n, k)
    for pos in (0, 1, 2, 3, 6, 7):
        args = list(ok)
        args[pos] = None
        assert L.mxq_gemm_mxfp4_out(*args) == mxq.ERR_NULL, pos
    for pos in (0, 4, 6, 7):
        args = list(ok)
        args[pos] = FAKE_ODD
        assert L.mxq_gemm_mxfp4_out(*args) == mxq.ERR_ALIGN, pos
    empty = list(ok)
    empty[8] = 0
    empty[0] = empty[6] = empty[7] = None
    assert L.mxq_gemm_mxfp4_out(*empty) == mxq.OK


def test_gemm_mxfp4_hadamard_out_validation():
    """Host-side checks of the fused GEMM -> transformed MXFP4 entry point (nothing is enqueued)."""
    L = mxq.lib()
    S = None
    # a0 as0 w0 ws0 bias epi mult yc ys M N K stream
    ok = [FAKE, FAKE, FAKE, FAKE, None, 1, FAKE, FAKE, FAKE, 512, 1024, 1024, S]
    bad_epi = list(ok)
    bad_epi[5] = 2
    assert L.mxq_gemm_mxfp4_hadamard_out(*bad_epi) == mxq.ERR_MODE
    for m, n, k in [(255, 1024, 1024), (512, 1024, 384), (512, 1000, 1024), (512, 1088, 1024), (512, 1024, 100)]:
        args = list(ok)
        args[9:12] = [m, n, k]
        assert L.mxq_gemm_mxfp4_hadamard_out(*args) == mxq.ERR_SHAPE, (m, n, k)
    for pos in (0, 1, 2, 3, 6, 7, 8):
        args = list(ok)
        args[pos] = None
        assert L.mxq_gemm_mxfp4_hadamard_out(*args) == mxq.ERR_NULL, pos
    for pos in (0, 4, 6, 7, 8):
        args = list(ok)
        args[pos] = FAKE_ODD
        assert L.mxq_gemm_mxfp4_hadamard_out(*args) == mxq.ERR_ALIGN, pos
    empty = list(ok)
    empty[9] = 0
    empty[0] = empty[6] = empty[7] = empty[8] = None
    assert L.mxq_gemm_mxfp4_hadamard_out(*empty) == mxq.OK


def test_gemm_fp8_static_out_validation():
    """Host-side checks of the fused W4A8 GEMM -> static FP8 entry point (nothing is enqueued)."""
    L = mxq.lib()
    S = None
    FAKE_F32_ODD = ctypes.c_void_p(0x10002)
    # a0 as0 w0 ws0 bias epi amax yc ys M N K stream
    ok = [FAKE, FAKE, FAKE, FAKE, None, 1, FAKE, FAKE, FAKE, 512, 1024, 1024, S]
    bad_epi = list(ok)
    bad_epi[5] = 3
    assert L.mxq_gemm_fp8_static_out(*bad_epi) == mxq.ERR_MODE
    # shapes the pipelined W4A8 kernel does not take
    for m, n, k in [(255, 1024, 1024), (512, 1024, 256), (512, 1020, 1024), (512, 1024, 100), (512, 1000, 1024)]:
        args = list(ok)
        args[9:12] = [m, n, k]
        assert L.mxq_gemm_fp8_static_out(*args) == mxq.ERR_SHAPE, (m, n, k)
    for pos in (0, 1, 2, 3, 6, 7, 8):
        args = list(ok)
        args[pos] = None
        assert L.mxq_gemm_fp8_static_out(*args) == mxq.ERR_NULL, pos
    for pos in (0, 4, 7, 8):
        args = list(ok)
        args[pos] = FAKE_ODD
        assert L.mxq_gemm_fp8_static_out(*args) == mxq.ERR_ALIGN, pos
    args = list(ok)
    args[6] = FAKE_F32_ODD
    assert L.mxq_gemm_fp8_static_out(*args) == mxq.ERR_ALIGN
    empty = list(ok)
    empty[10] = 0
    empty[0] = empty[6] = empty[7] = empty[8] = None
    assert L.mxq_gemm_fp8_static_out(*empty) == mxq.OK


def test_transform_validation():
    """Host-side checks of the transform_on entry points (nothing is enqueued)."""
    L = mxq.lib()
    S = None
    F4 = ctypes.c_void_p(0x10004)  # 4-byte aligned only
    # K must be a multiple of 128
    for k in (0, 32, 96, 160):
        assert L.mxq_quantize_mxfp4_hadamard(FAKE, 4, k, 256, FAKE, FAKE, FAKE, S) == mxq.ERR_SHAPE, k
        assert L.mxq_hadamard_channel_amax(FAKE, 4, k, 256, FAKE, S) == mxq.ERR_SHAPE, k
    assert L.mxq_quantize_mxfp4_hadamard(FAKE, 4, 128, 64, FAKE, FAKE, FAKE, S) == mxq.ERR_SHAPE  # ld < K
    for pos in (0, 4, 5, 6):
        args = [FAKE, 4, 128, 128, FAKE, FAKE, FAKE, S]
        args[pos] = None
        assert L.mxq_quantize_mxfp4_hadamard(*args) == mxq.ERR_NULL, pos
    for pos in (0, 4, 5, 6):
        args = [FAKE, 4, 128, 128, FAKE, FAKE, FAKE, S]
        args[pos] = FAKE_ODD if pos != 4 else F4
        assert L.mxq_quantize_mxfp4_hadamard(*args) == mxq.ERR_ALIGN, pos
    assert L.mxq_hadamard_channel_amax(None, 4, 128, 128, FAKE, S) == mxq.ERR_NULL
    assert L.mxq_hadamard_channel_amax(FAKE, 4, 128, 128, None, S) == mxq.ERR_NULL
    assert L.mxq_hadamard_channel_amax(FAKE, 4, 128, 132, FAKE, S) == mxq.ERR_ALIGN  # ld % 8
    for pos in (0, 1, 3, 4):
        args = [FAKE, FAKE, 128, FAKE, FAKE, S]
        args[pos] = None
        assert L.mxq_smoothquant_factors(*args) == mxq.ERR_NULL, pos
        args[pos] = ctypes.c_void_p(0x10002)
        assert L.mxq_smoothquant_factors(*args) == mxq.ERR_ALIGN, pos
    assert L.mxq_smoothquant_factors(FAKE, FAKE, -1, FAKE, FAKE, S) == mxq.ERR_SHAPE
    assert L.mxq_smoothquant_factors(None, None, 0, None, None, S) == mxq.OK
    assert L.mxq_quantize_mxfp4_hadamard(None, 0, 128, 128, None, None, None, S) == mxq.OK
    # qlinear on a transform_on block: mxq_qlinear refuses (no factors); the transform
    # entry point wants act_mult and K % 128 == 0
    p = mxq.Policy([[3, 0]])
    ws = mxq.qlinear_workspace_bytes(mxq.POLICY_TRANSFORM_ON, 4, 128)
    assert ws == mxq.qlinear_workspace_bytes(mxq.W4A4, 4, 128)
    assert L.mxq_qlinear(p.handle, 0, 0, FAKE, 4, 128, FAKE, FAKE, 8, None, 0, FAKE, FAKE, ws, S) == mxq.ERR_MODE
    assert L.mxq_qlinear_transform(p.handle, 0, 0, FAKE, 4, 128, FAKE, FAKE, 8, None, 0, None, FAKE, FAKE, ws,
                                   S) == mxq.ERR_NULL
    assert L.mxq_qlinear_transform(p.handle, 0, 0, FAKE, 4, 96, FAKE, FAKE, 8, None, 0, FAKE, FAKE, FAKE, ws,
                                   S) == mxq.ERR_SHAPE
    assert L.mxq_qlinear_transform(p.handle, 0, 0, FAKE, 4, 128, FAKE, FAKE, 8, None, 0, F4, FAKE, FAKE, ws,
                                   S) == mxq.ERR_ALIGN
    assert L.mxq_qlinear_transform(p.handle, 0, 0, FAKE, 4, 128, FAKE, FAKE, 8, None, 0, FAKE, FAKE, FAKE, ws - 1,
                                   S) == mxq.ERR_WORKSPACE
    p.close()


def test_selection_validation_and_host_policy_select():
    """Selector entry points: host-side checks, and the host-only rule ladder against the oracle."""
    import oracle

    L = mxq.lib()
    S = None
    F8 = ctypes.c_void_p(0x10004)  # not 8-byte aligned
    assert L.mxq_sqnr_accumulate(FAKE, FAKE, -1, FAKE, S) == mxq.ERR_SHAPE
    assert L.mxq_sqnr_accumulate(None, None, 0, None, S) == mxq.OK
    for pos in (0, 1, 3):
        args = [FAKE, FAKE, 64, FAKE, S]
        args[pos] = None
        assert L.mxq_sqnr_accumulate(*args) == mxq.ERR_NULL, pos
    assert L.mxq_sqnr_accumulate(FAKE_ODD, FAKE, 64, FAKE, S) == mxq.ERR_ALIGN
    assert L.mxq_sqnr_accumulate(FAKE, FAKE, 64, F8, S) == mxq.ERR_ALIGN
    # replay: shapes, nulls, workspace
    good = mxq.ReplayLinear(FAKE, FAKE, FAKE, 64, 96, 256)
    arr = (mxq.ReplayLinear * 2)(good, good)
    need = ctypes.c_size_t()
    assert L.mxq_replay_workspace_bytes(arr, 2, ctypes.byref(need)) == mxq.OK and need.value > 0
    bad_k = (mxq.ReplayLinear * 1)(mxq.ReplayLinear(FAKE, FAKE, FAKE, 64, 96, 96))
    assert L.mxq_replay_workspace_bytes(bad_k, 1, ctypes.byref(need)) == mxq.ERR_SHAPE
    assert L.mxq_block_replay_sqnr(bad_k, 1, FAKE, 1 << 30, FAKE, FAKE, S) == mxq.ERR_SHAPE
    null_w = (mxq.ReplayLinear * 1)(mxq.ReplayLinear(FAKE, None, FAKE, 64, 96, 256))
    assert L.mxq_block_replay_sqnr(null_w, 1, FAKE, 1 << 30, FAKE, FAKE, S) == mxq.ERR_NULL
    odd = (mxq.ReplayLinear * 1)(mxq.ReplayLinear(FAKE, FAKE, FAKE_ODD, 64, 96, 256))
    assert L.mxq_block_replay_sqnr(odd, 1, FAKE, 1 << 30, FAKE, FAKE, S) == mxq.ERR_ALIGN
    assert L.mxq_block_replay_sqnr(arr, 2, FAKE, 16, FAKE, FAKE, S) == mxq.ERR_WORKSPACE
    assert L.mxq_block_replay_sqnr(arr, 2, None, 1 << 30, FAKE, FAKE, S) == mxq.ERR_WORKSPACE
    assert L.mxq_block_replay_sqnr(arr, 2, FAKE, 1 << 30, None, FAKE, S) == mxq.ERR_NULL
    assert L.mxq_block_replay_sqnr(arr, 2, FAKE, 1 << 30, FAKE, F8, S) == mxq.ERR_ALIGN
    assert L.mxq_block_replay_sqnr(arr, -1, FAKE, 1 << 30, FAKE, FAKE, S) == mxq.ERR_SHAPE
    assert L.mxq_block_replay_sqnr(None, 0, None, 0, None, None, S) == mxq.OK
    # the rule ladder (host only) against the oracle, on random sums and on exact 10 dB steps
    g = np.random.default_rng(3)
    sig = np.ldexp(g.uniform(1, 2, (2, 40)), g.integers(0, 40, (2, 40)))
    off = np.stack([sig, sig * 10.0 ** (-g.uniform(0.5, 4.0, (2, 40)))], axis=2)
    on = np.stack([sig, sig * 10.0 ** (-g.uniform(0.5, 4.0, (2, 40)))], axis=2)
    off[0, 0, 1] = 0.0   # no noise: +inf dB
    on[1, 3, 0] = 0.0    # no signal: -inf dB
    off[1, 5] = [100.0, 10.0]    # exactly 10 dB: the mid tier's floor is not crossed
    on[1, 5] = [100.0, 10.0]
    for tier, name in ((mxq.TIER_LOW, "low"), (mxq.TIER_MID, "mid"), (mxq.TIER_HIGH, "high")):
        got = mxq.policy_select(off, on, tier)
        db = lambda a: np.vectorize(oracle.sqnr_db)(a[..., 0], a[..., 1])
        want = oracle.select_policy(db(off), db(on), name)
        assert np.array_equal(got, want), name
    assert mxq.policy_select(off, on, mxq.TIER_MID)[1, 5] == mxq.W4A8
    with pytest.raises(mxq.MxqError):
        mxq.policy_select(off, on, 3)


def test_lowrank_validation():
    """Host-side checks of the SVDQuant branch entry points (nothing is enqueued)."""
    L = mxq.lib()
    S = None
    for r in (0, 16, 48, 160, -32):
        assert L.mxq_lowrank_down(FAKE, 64, 256, FAKE, r, FAKE, S) == mxq.ERR_SHAPE, r
        assert L.mxq_lowrank_up(FAKE, FAKE, FAKE, 64, 256, r, 0, FAKE, S) == mxq.ERR_SHAPE, r
    assert L.mxq_lowrank_down(FAKE, 64, 96, FAKE, 32, FAKE, S) == mxq.ERR_SHAPE  # K % 128
    assert L.mxq_lowrank_down(FAKE, 64, 192, FAKE, 32, FAKE, S) == mxq.ERR_SHAPE
    assert L.mxq_lowrank_up(FAKE, FAKE, FAKE, 64, 48, 32, 0, FAKE, S) == mxq.ERR_SHAPE  # N % 32
    assert L.mxq_lowrank_up(FAKE, FAKE, FAKE, 64, 256, 32, 2, FAKE, S) == mxq.ERR_MODE
    for pos in (0, 3, 5):
        args = [FAKE, 64, 256, FAKE, 32, FAKE, S]
        args[pos] = None
        assert L.mxq_lowrank_down(*args) == mxq.ERR_NULL, pos
        args[pos] = FAKE_ODD
        assert L.mxq_lowrank_down(*args) == mxq.ERR_ALIGN, pos
    for pos in (0, 1, 2, 7):
        args = [FAKE, FAKE, FAKE, 64, 256, 32, 0, FAKE, S]
        args[pos] = None
        assert L.mxq_lowrank_up(*args) == mxq.ERR_NULL, pos
        args[pos] = FAKE_ODD
        assert L.mxq_lowrank_up(*args) == mxq.ERR_ALIGN, pos
    assert L.mxq_lowrank_down(None, 0, 256, None, 32, None, S) == mxq.OK
    assert L.mxq_lowrank_up(None, None, None, 0, 256, 32, 0, None, S) == mxq.OK


def test_quantize_act_lowrank_validation():
    """Host-side checks of the quantizer fused with the branch's first half (nothing is enqueued)."""
    L = mxq.lib()
    S = None
    # x0 M1 K2 l1t3 r4 codes5 scales6 t7 stream
    ok = [FAKE, 64, 256, FAKE, 32, FAKE, FAKE, FAKE, S]
    for r in (0, 16, 48, 160, -32):
        args = list(ok)
        args[4] = r
        assert L.mxq_quantize_act_lowrank(*args) == mxq.ERR_SHAPE, r
    for k in (96, 192, 100):
        args = list(ok)
        args[2] = k
        assert L.mxq_quantize_act_lowrank(*args) == mxq.ERR_SHAPE, k
    for pos in (0, 3, 5, 6, 7):
        args = list(ok)
        args[pos] = None
        assert L.mxq_quantize_act_lowrank(*args) == mxq.ERR_NULL, pos
        args[pos] = FAKE_ODD
        assert L.mxq_quantize_act_lowrank(*args) == mxq.ERR_ALIGN, pos
    assert L.mxq_quantize_act_lowrank(None, 0, 256, None, 32, None, None, None, S) == mxq.OK


def test_gemm_lowrank_validation():
    """Host-side checks of the GEMM with the branch in its sums; every case is refused before any
    launch (the valid argument list itself is never passed)."""
    L = mxq.lib()
    S = None
    # a0 as1 w2 ws3 bias4 t5 l2_6 r7 epi8 y9 ys10 M11 N12 K13 stream
    ok = [FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 32, 0, FAKE, None, 512, 1024, 1024, S]

    def call(**chg):
        args = list(ok)
        for pos, v in chg.items():
            args[int(pos[1:])] = v
        return L.mxq_gemm_lowrank(*args)

    assert call(p8=2) == mxq.ERR_MODE
    for r in (0, 16, 48, 160, -32):
        assert call(p7=r) == mxq.ERR_SHAPE, r
    assert call(p13=100) == mxq.ERR_SHAPE
    # shapes the pipelined kernel does not take; N % 128 for the MXFP4 output
    for m, n, k in [(255, 1024, 1024), (512, 1024, 384), (512, 1004, 1024)]:
        assert call(p11=m, p12=n, p13=k) == mxq.ERR_SHAPE, (m, n, k)
        assert call(p11=m, p12=n, p13=k, p10=FAKE) == mxq.ERR_SHAPE, (m, n, k)
    assert call(p12=1088, p10=FAKE) == mxq.ERR_SHAPE
    for pos in (0, 1, 2, 3, 5, 6, 9):
        assert call(**{f"p{pos}": None}) == mxq.ERR_NULL, pos
        assert call(**{f"p{pos}": None, "p10": FAKE}) == mxq.ERR_NULL, pos
    for pos in (0, 1, 2, 3, 4, 5, 6, 9):
        assert call(**{f"p{pos}": FAKE_ODD}) == mxq.ERR_ALIGN, pos
    assert call(p10=FAKE_ODD) == mxq.ERR_ALIGN
    assert call(p11=0, p0=None, p5=None, p9=None) == mxq.OK


def test_static_fp8_validation():
    """Host-side checks of the static FP8 quantizer and its calibration (nothing is enqueued)."""
    L = mxq.lib()
    S = None
    FAKE_F32_ODD = ctypes.c_void_p(0x10002)  # not 4-byte aligned
    # x M K ld codes scales
    for k in (0, 16, 48):
        assert L.mxq_quantize_act_fp8_static(FAKE, 4, k, 64, FAKE, FAKE, FAKE, S) == mxq.ERR_SHAPE
        assert L.mxq_fp8_calibrate(FAKE, 4, k, 64, FAKE, S) == mxq.ERR_SHAPE
    assert L.mxq_quantize_act_fp8_static(FAKE, 4, 64, 32, FAKE, FAKE, FAKE, S) == mxq.ERR_SHAPE  # ld < K
    assert L.mxq_fp8_calibrate(FAKE, -1, 64, 64, FAKE, S) == mxq.ERR_SHAPE
    for pos in (0, 4, 5, 6):
        args = [FAKE, 4, 64, 64, FAKE, FAKE, FAKE, S]
        args[pos] = None
        assert L.mxq_quantize_act_fp8_static(*args) == mxq.ERR_NULL, pos
    assert L.mxq_fp8_calibrate(None, 4, 64, 64, FAKE, S) == mxq.ERR_NULL
    assert L.mxq_fp8_calibrate(FAKE, 4, 64, 64, None, S) == mxq.ERR_NULL
    assert L.mxq_quantize_act_fp8_static(FAKE_ODD, 4, 64, 64, FAKE, FAKE, FAKE, S) == mxq.ERR_ALIGN
    assert L.mxq_quantize_act_fp8_static(FAKE, 4, 64, 64, FAKE_F32_ODD, FAKE, FAKE, S) == mxq.ERR_ALIGN
    assert L.mxq_quantize_act_fp8_static(FAKE, 4, 64, 68, FAKE, FAKE, FAKE, S) == mxq.ERR_ALIGN  # ld % 8
    assert L.mxq_fp8_calibrate(FAKE_ODD, 4, 64, 64, FAKE, S) == mxq.ERR_ALIGN
    assert L.mxq_fp8_calibrate(FAKE, 4, 64, 64, FAKE_F32_ODD, S) == mxq.ERR_ALIGN
    # empty inputs enqueue nothing
    assert L.mxq_quantize_act_fp8_static(None, 0, 64, 64, None, None, None, S) == mxq.OK
    assert L.mxq_fp8_calibrate(None, 0, 64, 64, None, S) == mxq.OK


def test_policy_table_roundtrip_and_errors():
    table = np.array([[0, 1, 0], [1, 1, 0]], np.uint8)
    p = mxq.Policy(table)
    for e in range(2):
        for b in range(3):
            assert p.mode(e, b) == table[e, b]
    for e, b in ((2, 0), (0, 3), (-1, 0), (0, -1)):
        with pytest.raises(mxq.MxqError) as ei:
            p.mode(e, b)
        assert ei.value.status == mxq.ERR_RANGE
    p.close()
    # transform_on is a policy value (W4A4 with the Hadamard + SmoothQuant transform); bf16 is not
    pt = mxq.Policy([[3, 0]])
    assert pt.mode(0, 0) == mxq.POLICY_TRANSFORM_ON
    pt.close()
    for bad in ([[0, 2]], [[4, 0]], [[9]]):
        with pytest.raises(mxq.MxqError) as ei:
            mxq.Policy(bad)
        assert ei.value.status == mxq.ERR_MODE
    h = ctypes.c_void_p()
    assert mxq.lib().mxq_policy_create(None, 1, 1, ctypes.byref(h)) == mxq.ERR_NULL
    assert mxq.lib().mxq_policy_create(table.ctypes.data_as(ctypes.c_void_p), 0, 3, ctypes.byref(h)) == mxq.ERR_SHAPE
    assert mxq.lib().mxq_policy_destroy(None) == mxq.OK


def test_workspace_bytes_and_qlinear_validation():
    assert mxq.qlinear_workspace_bytes(mxq.W4A4, 256, 512) == 256 * 256 + 256 * 16
    assert mxq.qlinear_workspace_bytes(mxq.W4A8, 256, 512) == 256 * 512 + 1024
    assert mxq.qlinear_workspace_bytes(mxq.W4A8, 3, 32) == 256 + 256
    with pytest.raises(mxq.MxqError):
        mxq.qlinear_workspace_bytes(mxq.POLICY_BF16, 4, 64)
    L = mxq.lib()
    p = mxq.Policy([[0, 1]])
    S = None
    ws_small = mxq.qlinear_workspace_bytes(mxq.W4A8, 4, 64) - 1
    # W4A8 block with a workspace one byte short
    assert L.mxq_qlinear(p.handle, 0, 1, FAKE, 4, 64, FAKE, FAKE, 8, None, 0, FAKE, FAKE, ws_small, S) \
        == mxq.ERR_WORKSPACE
    assert L.mxq_qlinear(p.handle, 0, 0, FAKE, 4, 64, FAKE, FAKE, 8, None, 0, FAKE, None, 1 << 20, S) \
        == mxq.ERR_WORKSPACE
    assert L.mxq_qlinear(p.handle, 1, 0, FAKE, 4, 64, FAKE, FAKE, 8, None, 0, FAKE, FAKE, 1 << 20, S) \
        == mxq.ERR_RANGE
    assert L.mxq_qlinear(None, 0, 0, FAKE, 4, 64, FAKE, FAKE, 8, None, 0, FAKE, FAKE, 1 << 20, S) \
        == mxq.ERR_NULL
    assert L.mxq_qlinear(p.handle, 0, 0, FAKE, 4, 64, FAKE, FAKE, 8, None, 5, FAKE, FAKE, 1 << 20, S) \
        == mxq.ERR_MODE
    assert L.mxq_qlinear(p.handle, 0, 0, FAKE, 0, 64, None, None, 8, None, 0, None, None, 0, S) == mxq.OK
    p.close()


def test_python_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    with pytest.raises(TypeError):
        mxq.quantize_weight_mxfp4(torch.zeros((4, 64), dtype=torch.bfloat16))


def test_gemm_kernel_selection():
    """The pipelined kernel takes the workload shapes; everything else the direct kernel."""
    pipe = [(0, 75600, 5120, 5120), (0, 75600, 13824, 5120), (1, 75600, 5120, 13824), (0, 32760, 15360, 5120),
            (1, 11440, 3072, 14336), (0, 512, 5120, 5120), (0, 256, 256, 512), (1, 256, 256, 384),
            (0, 75600, 15360, 5120), (1, 111600, 13824, 5120)]   # outputs past 2 GiB (addressed per tile)
    direct = [(0, 255, 512, 512),     # M below one tile
              (0, 512, 260, 512),     # N not a multiple of 8
              (0, 512, 512, 384),     # fewer stages than the W4A4 ring
              (1, 512, 512, 256),     # fewer stages than the W4A8 ring
              (0, 512, 512, 544),     # K not a multiple of 128
              (1, 170000, 512, 13824),  # FP8 activation codes of 2^31 bytes or more
              (0, 512, 300000, 16384)]  # packed weight of 2^31 bytes or more
    # the MXFP4 output is addressed as a whole: below 2^31 bytes
    assert mxq.gemm_mxfp4_out_supported(75600, 13824, 5120)
    assert not mxq.gemm_mxfp4_out_supported(200000, 22528, 512)
    assert mxq.lib().mxq_gemm_mxfp4_out(FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, FAKE, 200000, 22528, 512,
                                        None) == mxq.ERR_SHAPE
    for mode, m, n, k in pipe:
        assert mxq.gemm_kernel_name(mode, m, n, k).startswith("pipe_"), (mode, m, n, k)
    for mode, m, n, k in direct:
        assert mxq.gemm_kernel_name(mode, m, n, k).startswith("direct_"), (mode, m, n, k)
    assert mxq.gemm_kernel_name(2, 512, 512, 512) == "invalid"
