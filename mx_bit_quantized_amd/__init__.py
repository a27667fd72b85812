"""mx_bit_quantized_amd - MI355X-native W4A4 / W4A8 MX quantized linear.

Thin Python binding over libmxq.so (include/mxq.h): argument marshalling
only. Every step of the computation runs in the library's gfx950 kernels;
torch supplies device memory and the current HIP stream. There is no CPU or
PyTorch fallback: if the library is missing, every call raises.

Names mirror the C ABI without its ``mxq_`` prefix:

    quantize_weight_mxfp4(w)                      -> (codes, scales)
    quantize_act(mode, x)                         -> (codes, scales)
    gemm(mode, a_codes, a_scales, w_codes, w_scales, bias=None, epilogue=EPI_NONE)
    gemm_kernel_name(mode, M, N, K)
    mxfp4_to_canonical(codes, scales, rows, K) / mxfp4_from_canonical(codes_rm, scales_rm)
    Policy(table) / policy_create / policy_destroy / policy_mode
    qlinear_workspace_bytes(mode, M, K)
    qlinear(policy, expert, block, x, w_codes, w_scales, bias=None, epilogue=EPI_NONE)
    qlinear_noalloc(policy, expert, block, x, w_codes, w_scales, y, bias=None, epilogue=EPI_NONE)
"""

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxq.so")

# status codes, modes and epilogues (include/mxq.h)
OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_MODE, ERR_WORKSPACE, ERR_HIP, ERR_RANGE, ERR_SCRATCH, ERR_NONFINITE = range(10)
NOALLOC_SCRATCH_BYTES = 64 << 20  # MXQ_NOALLOC_SCRATCH_BYTES
W4A4, W4A8, POLICY_BF16, POLICY_TRANSFORM_ON = 0, 1, 2, 3
TIER_LOW, TIER_MID, TIER_HIGH = 0, 1, 2
EPI_NONE, EPI_GELU_TANH = 0, 1

# every function the header declares, with its ctypes signature
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32


class ReplayLinear(ctypes.Structure):
    """mxq_replay_linear: one linear of a block replay (device pointers, sizes)."""
    _fields_ = [("x", _P), ("w", _P), ("y_ref", _P), ("M", _I64), ("N", _I64), ("K", _I64)]

_SIGS = {
    "mxq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "mxq_version": (ctypes.c_int, []),
    "mxq_quantize_weight_mxfp4": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _P, _P]),
    "mxq_quantize_act": (ctypes.c_int, [ctypes.c_int, _P, _I64, _I64, _I64, _P, _P, _P]),
    "mxq_fp8_calibrate": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _P]),
    "mxq_lowrank_down": (ctypes.c_int, [_P, _I64, _I64, _P, _I64, _P, _P]),
    "mxq_lowrank_up": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, ctypes.c_int, _P, _P]),
    "mxq_quantize_act_lowrank": (ctypes.c_int, [_P, _I64, _I64, _P, _I64, _P, _P, _P, _P]),
    "mxq_gemm_lowrank": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I64, ctypes.c_int, _P, _P, _I64, _I64, _I64,
                                        _P]),
    "mxq_sqnr_accumulate": (ctypes.c_int, [_P, _P, _I64, _P, _P]),
    "mxq_replay_workspace_bytes": (ctypes.c_int, [_P, _I32, ctypes.POINTER(ctypes.c_size_t)]),
    "mxq_block_replay_sqnr": (ctypes.c_int, [_P, _I32, _P, ctypes.c_size_t, _P, _P, _P]),
    "mxq_policy_select": (ctypes.c_int, [_P, _P, _I32, _I32, _I32, _P]),
    "mxq_hadamard_channel_amax": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _P]),
    "mxq_smoothquant_factors": (ctypes.c_int, [_P, _P, _I64, _P, _P, _P]),
    "mxq_quantize_mxfp4_hadamard": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "mxq_quantize_act_fp8_static": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "mxq_gemm": (ctypes.c_int, [ctypes.c_int, _P, _P, _P, _P, _P, ctypes.c_int, _P, _I64, _I64, _I64, _P]),
    "mxq_gemm_mxfp4_out": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.c_int, _P, _P, _I64, _I64, _I64, _P]),
    "mxq_gemm_mxfp4_hadamard_out": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.c_int, _P, _P, _P, _I64, _I64,
                                                    _I64, _P]),
    "mxq_gemm_fp8_static_out": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.c_int, _P, _P, _P, _I64, _I64, _I64,
                                                _P]),
    "mxq_gemm_kernel_name": (ctypes.c_char_p, [ctypes.c_int, _I64, _I64, _I64]),
    "mxq_mxfp4_to_canonical": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _P, _P]),
    "mxq_mxfp4_from_canonical": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _P, _P]),
    "mxq_policy_create": (ctypes.c_int, [_P, _I32, _I32, ctypes.POINTER(_P)]),
    "mxq_policy_destroy": (ctypes.c_int, [_P]),
    "mxq_policy_mode": (ctypes.c_int, [_P, _I32, _I32, ctypes.POINTER(ctypes.c_int)]),
    "mxq_qlinear_workspace_bytes": (ctypes.c_int, [ctypes.c_int, _I64, _I64, ctypes.POINTER(ctypes.c_size_t)]),
    "mxq_qlinear": (ctypes.c_int, [_P, _I32, _I32, _P, _I64, _I64, _P, _P, _I64, _P, ctypes.c_int, _P,
                                   _P, ctypes.c_size_t, _P]),
    "mxq_qlinear_transform": (ctypes.c_int, [_P, _I32, _I32, _P, _I64, _I64, _P, _P, _I64, _P, ctypes.c_int, _P,
                                             _P, _P, ctypes.c_size_t, _P]),
    "mxq_qlinear_noalloc": (ctypes.c_int, [_P, _I32, _I32, _P, _I64, _I64, _P, _P, _I64, _P, ctypes.c_int, _P, _P]),
}


class MxqError(RuntimeError):
    def __init__(self, status, what):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


_lib = None


def lib():
    """The loaded libmxq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m mx_bit_quantized_amd._build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status):
    return lib().mxq_status_string(int(status)).decode()


def version():
    return lib().mxq_version()


def _check(status, what):
    if status != OK:
        raise MxqError(status, what)


# ------------------------------------------------------------- tensors ----

def _torch():
    import torch

    return torch


def _stream_handle(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dev_ptr(t, name, dtype=None):
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (no implicit copies)")
    return ctypes.c_void_p(t.data_ptr()) if t.numel() else None


def _rows_k(t, name):
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D [rows, K]")
    return int(t.shape[0]), int(t.shape[1])


def mx_scale_shape(rows, K):
    """Shape of group-major MXFP4 scales: [ceil(K/128), rows, 4] bytes."""
    return ((K + 127) // 128, rows, 4)


def act_buffers(mode, M, K, device):
    """Empty (codes, scales) tensors for quantize_act in ``mode``.

    MXFP4 codes are a byte buffer shaped [M, K/2] whose contents are laid out
    in K-panels of 128 elements (include/mxq.h); FP8 codes are row-major [M, K].
    """
    torch = _torch()
    if mode == W4A4:
        return (torch.empty((M, K // 2), dtype=torch.uint8, device=device),
                torch.empty(mx_scale_shape(M, K), dtype=torch.uint8, device=device))
    if mode == W4A8:
        return (torch.empty((M, K), dtype=torch.uint8, device=device),
                torch.empty((M,), dtype=torch.float32, device=device))
    raise MxqError(ERR_MODE, "act_buffers")


def quantize_weight_mxfp4(w, codes=None, scales=None, stream=None):
    """RTN MXFP4 packing of bf16 weights [N, K] -> (codes, scales).

    codes: uint8 tensor of N * K/2 bytes, shaped [N, K/2] but laid out in
    K-panels of 128 elements (include/mxq.h); scales: uint8 [ceil(K/128), N, 4].
    """
    torch = _torch()
    n, k = _rows_k(w, "w")
    if codes is None:
        codes = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty(mx_scale_shape(n, k), dtype=torch.uint8, device=w.device)
    st = lib().mxq_quantize_weight_mxfp4(_dev_ptr(w, "w", torch.bfloat16), n, k, k,
                                          _dev_ptr(codes, "codes", torch.uint8),
                                          _dev_ptr(scales, "scales", torch.uint8), _stream_handle(stream))
    _check(st, "quantize_weight_mxfp4")
    return codes, scales


def quantize_act(mode, x, codes=None, scales=None, stream=None):
    """Dynamic activation quantization of bf16 x [M, K] in ``mode`` -> (codes, scales)."""
    torch = _torch()
    m, k = _rows_k(x, "x")
    if codes is None or scales is None:
        codes, scales = act_buffers(mode, m, k, x.device) if mode in (W4A4, W4A8) else (None, None)
    st = lib().mxq_quantize_act(int(mode), _dev_ptr(x, "x", torch.bfloat16), m, k, k,
                                 _dev_ptr(codes, "codes"), _dev_ptr(scales, "scales"), _stream_handle(stream))
    _check(st, "quantize_act")
    return codes, scales


def fp8_calibrate(x, amax=None, stream=None):
    """Fold bf16 x [M, K] into a running amax (device float32 [1], created as 0 when None) -> amax."""
    torch = _torch()
    m, k = _rows_k(x, "x")
    if amax is None:
        amax = torch.zeros((1,), dtype=torch.float32, device=x.device)
    st = lib().mxq_fp8_calibrate(_dev_ptr(x, "x", torch.bfloat16), m, k, k, _dev_ptr(amax, "amax", torch.float32),
                                  _stream_handle(stream))
    _check(st, "fp8_calibrate")
    return amax


def quantize_act_fp8_static(x, amax, codes=None, scales=None, stream=None):
    """Static FP8 quantization of bf16 x [M, K] with the calibrated amax (device float32 [1]) -> (codes, scales)."""
    torch = _torch()
    m, k = _rows_k(x, "x")
    if codes is None or scales is None:
        codes, scales = act_buffers(W4A8, m, k, x.device)
    st = lib().mxq_quantize_act_fp8_static(_dev_ptr(x, "x", torch.bfloat16), m, k, k,
                                            _dev_ptr(amax, "amax", torch.float32), _dev_ptr(codes, "codes"),
                                            _dev_ptr(scales, "scales"), _stream_handle(stream))
    _check(st, "quantize_act_fp8_static")
    return codes, scales


def hadamard_channel_amax(x, amax=None, stream=None):
    """Fold bf16 x [M, K] into the running per-channel max |transform(x)| (device float32 [K]) -> amax."""
    torch = _torch()
    m, k = _rows_k(x, "x")
    if amax is None:
        amax = torch.zeros((k,), dtype=torch.float32, device=x.device)
    st = lib().mxq_hadamard_channel_amax(_dev_ptr(x, "x", torch.bfloat16), m, k, k,
                                          _dev_ptr(amax, "amax", torch.float32), _stream_handle(stream))
    _check(st, "hadamard_channel_amax")
    return amax


def smoothquant_factors(act_amax, w_amax, act_mult=None, w_mult=None, stream=None):
    """SmoothQuant factor vectors (act_mult, w_mult), device float32 [K], from the two rotated maxima."""
    torch = _torch()
    k = int(act_amax.numel())
    if act_mult is None:
        act_mult = torch.empty((k,), dtype=torch.float32, device=act_amax.device)
    if w_mult is None:
        w_mult = torch.empty((k,), dtype=torch.float32, device=act_amax.device)
    st = lib().mxq_smoothquant_factors(_dev_ptr(act_amax, "act_amax", torch.float32),
                                        _dev_ptr(w_amax, "w_amax", torch.float32), k,
                                        _dev_ptr(act_mult, "act_mult", torch.float32),
                                        _dev_ptr(w_mult, "w_mult", torch.float32), _stream_handle(stream))
    _check(st, "smoothquant_factors")
    return act_mult, w_mult


def quantize_mxfp4_hadamard(x, mult, codes=None, scales=None, stream=None):
    """MXFP4 of the transformed bf16 x [M, K] (rotation, channel factor ``mult``, bf16) -> (codes, scales)."""
    torch = _torch()
    m, k = _rows_k(x, "x")
    if codes is None or scales is None:
        codes, scales = act_buffers(W4A4, m, k, x.device)
    st = lib().mxq_quantize_mxfp4_hadamard(_dev_ptr(x, "x", torch.bfloat16), m, k, k,
                                            _dev_ptr(mult, "mult", torch.float32), _dev_ptr(codes, "codes"),
                                            _dev_ptr(scales, "scales"), _stream_handle(stream))
    _check(st, "quantize_mxfp4_hadamard")
    return codes, scales


def gemm(mode, a_codes, a_scales, w_codes, w_scales, bias=None, epilogue=EPI_NONE, y=None, stream=None):
    """Scaled GEMM on quantized operands -> y bf16 [M, N]."""
    torch = _torch()
    m = int(a_codes.shape[0])
    n = int(w_codes.shape[0])
    k = int(w_codes.shape[1]) * 2
    if y is None:
        y = torch.empty((m, n), dtype=torch.bfloat16, device=w_codes.device)
    st = lib().mxq_gemm(int(mode), _dev_ptr(a_codes, "a_codes"), _dev_ptr(a_scales, "a_scales"),
                         _dev_ptr(w_codes, "w_codes", torch.uint8), _dev_ptr(w_scales, "w_scales", torch.uint8),
                         _dev_ptr(bias, "bias", torch.bfloat16), int(epilogue),
                         _dev_ptr(y, "y", torch.bfloat16), m, n, k, _stream_handle(stream))
    _check(st, "gemm")
    return y


def gemm_mxfp4_out(a_codes, a_scales, w_codes, w_scales, bias=None, epilogue=EPI_NONE, y_codes=None,
                   y_scales=None, stream=None):
    """W4A4 GEMM whose output is quantized straight to the W4A4 activation format.

    Returns (y_codes, y_scales), equal to quantize_act(W4A4, gemm(W4A4, ...)).
    """
    torch = _torch()
    m = int(a_codes.shape[0])
    n = int(w_codes.shape[0])
    k = int(w_codes.shape[1]) * 2
    if y_codes is None or y_scales is None:
        y_codes, y_scales = act_buffers(W4A4, m, n, w_codes.device)
    st = lib().mxq_gemm_mxfp4_out(_dev_ptr(a_codes, "a_codes"), _dev_ptr(a_scales, "a_scales"),
                                   _dev_ptr(w_codes, "w_codes", torch.uint8),
                                   _dev_ptr(w_scales, "w_scales", torch.uint8),
                                   _dev_ptr(bias, "bias", torch.bfloat16), int(epilogue),
                                   _dev_ptr(y_codes, "y_codes", torch.uint8),
                                   _dev_ptr(y_scales, "y_scales", torch.uint8), m, n, k, _stream_handle(stream))
    _check(st, "gemm_mxfp4_out")
    return y_codes, y_scales


def gemm_mxfp4_hadamard_out(a_codes, a_scales, w_codes, w_scales, mult, bias=None, epilogue=EPI_NONE,
                            y_codes=None, y_scales=None, stream=None):
    """W4A4 GEMM whose output is quantized straight to the transform_on activation of a next layer.

    Returns (y_codes, y_scales), equal to quantize_mxfp4_hadamard(gemm(W4A4, ...), mult); mult is
    the next layer's act_mult (float32 [N]). Same shapes as gemm_mxfp4_out.
    """
    torch = _torch()
    m = int(a_codes.shape[0])
    n = int(w_codes.shape[0])
    k = int(w_codes.shape[1]) * 2
    if y_codes is None or y_scales is None:
        y_codes, y_scales = act_buffers(W4A4, m, n, w_codes.device)
    st = lib().mxq_gemm_mxfp4_hadamard_out(_dev_ptr(a_codes, "a_codes"), _dev_ptr(a_scales, "a_scales"),
                                            _dev_ptr(w_codes, "w_codes", torch.uint8),
                                            _dev_ptr(w_scales, "w_scales", torch.uint8),
                                            _dev_ptr(bias, "bias", torch.bfloat16), int(epilogue),
                                            _dev_ptr(mult, "mult", torch.float32),
                                            _dev_ptr(y_codes, "y_codes", torch.uint8),
                                            _dev_ptr(y_scales, "y_scales", torch.uint8), m, n, k,
                                            _stream_handle(stream))
    _check(st, "gemm_mxfp4_hadamard_out")
    return y_codes, y_scales


def gemm_mxfp4_out_supported(M, N, K):
    """Whether gemm_mxfp4_out takes (M, N, K): the pipelined kernel's shapes with N % 128 == 0 and
    an MXFP4 output below 2 GiB."""
    return gemm_kernel_name(W4A4, M, N, K).startswith("pipe_") and N % 128 == 0 and M * (N // 2) < 2 ** 31 - 256


def gemm_fp8_static_out(a_codes, a_scales, w_codes, w_scales, out_amax, bias=None, epilogue=EPI_NONE,
                        y_codes=None, y_scales=None, stream=None):
    """W4A8 GEMM whose output is quantized straight to static FP8 with the calibrated ``out_amax``.

    Returns (y_codes, y_scales), equal to quantize_act_fp8_static(gemm(W4A8, ...), out_amax).
    """
    torch = _torch()
    m = int(a_codes.shape[0])
    n = int(w_codes.shape[0])
    k = int(w_codes.shape[1]) * 2
    if y_codes is None or y_scales is None:
        y_codes, y_scales = act_buffers(W4A8, m, n, w_codes.device)
    st = lib().mxq_gemm_fp8_static_out(_dev_ptr(a_codes, "a_codes"), _dev_ptr(a_scales, "a_scales"),
                                        _dev_ptr(w_codes, "w_codes", torch.uint8),
                                        _dev_ptr(w_scales, "w_scales", torch.uint8),
                                        _dev_ptr(bias, "bias", torch.bfloat16), int(epilogue),
                                        _dev_ptr(out_amax, "out_amax", torch.float32),
                                        _dev_ptr(y_codes, "y_codes", torch.uint8),
                                        _dev_ptr(y_scales, "y_scales", torch.float32), m, n, k,
                                        _stream_handle(stream))
    _check(st, "gemm_fp8_static_out")
    return y_codes, y_scales


def gemm_fp8_static_out_supported(M, N, K):
    """Whether gemm_fp8_static_out takes (M, N, K): the pipelined W4A8 kernel's shapes with N % 32 == 0."""
    return gemm_kernel_name(W4A8, M, N, K).startswith("pipe_") and N % 32 == 0


def gemm_kernel_name(mode, M, N, K):
    """Name of the kernel gemm() runs for this mode and shape (host query)."""
    return lib().mxq_gemm_kernel_name(int(mode), int(M), int(N), int(K)).decode()


# ------------------------------------------------------------- layouts ----

def mxfp4_to_canonical(codes, scales, rows, K, codes_rm=None, scales_rm=None, stream=None):
    """Library MXFP4 layout -> canonical OCP row-major: (codes_rm uint8 [rows, K/2], scales_rm uint8 [rows, K/32])."""
    torch = _torch()
    if codes_rm is None:
        codes_rm = torch.empty((rows, K // 2), dtype=torch.uint8, device=codes.device)
    if scales_rm is None:
        scales_rm = torch.empty((rows, K // 32), dtype=torch.uint8, device=codes.device)
    st = lib().mxq_mxfp4_to_canonical(_dev_ptr(codes, "codes", torch.uint8), _dev_ptr(scales, "scales", torch.uint8),
                                       int(rows), int(K), _dev_ptr(codes_rm, "codes_rm", torch.uint8),
                                       _dev_ptr(scales_rm, "scales_rm", torch.uint8), _stream_handle(stream))
    _check(st, "mxfp4_to_canonical")
    return codes_rm, scales_rm


def mxfp4_from_canonical(codes_rm, scales_rm, codes=None, scales=None, stream=None):
    """Canonical OCP row-major MXFP4 ([rows, K/2], [rows, K/32]) -> library layout (codes, scales)."""
    torch = _torch()
    rows, half = _rows_k(codes_rm, "codes_rm")
    k = 2 * half
    if codes is None:
        codes = torch.empty((rows, half), dtype=torch.uint8, device=codes_rm.device)
    if scales is None:
        scales = torch.empty(mx_scale_shape(rows, k), dtype=torch.uint8, device=codes_rm.device)
    st = lib().mxq_mxfp4_from_canonical(_dev_ptr(codes_rm, "codes_rm", torch.uint8),
                                         _dev_ptr(scales_rm, "scales_rm", torch.uint8), rows, k,
                                         _dev_ptr(codes, "codes", torch.uint8), _dev_ptr(scales, "scales", torch.uint8),
                                         _stream_handle(stream))
    _check(st, "mxfp4_from_canonical")
    return codes, scales


# -------------------------------------------------------------- policy ----

def policy_create(table):
    t = np.ascontiguousarray(np.asarray(table, dtype=np.uint8))
    if t.ndim != 2:
        raise ValueError("policy table must be 2-D [n_experts, n_blocks]")
    h = ctypes.c_void_p()
    st = lib().mxq_policy_create(t.ctypes.data_as(ctypes.c_void_p), t.shape[0], t.shape[1], ctypes.byref(h))
    _check(st, "policy_create")
    return h


def policy_destroy(handle):
    _check(lib().mxq_policy_destroy(handle), "policy_destroy")


def policy_mode(handle, expert, block):
    mode = ctypes.c_int()
    _check(lib().mxq_policy_mode(handle, int(expert), int(block), ctypes.byref(mode)), "policy_mode")
    return mode.value


class Policy:
    """Per-expert, per-block W4A4 / W4A8 table owned by the library."""

    def __init__(self, table):
        self.table = np.array(table, dtype=np.uint8)
        self.handle = policy_create(self.table)

    def mode(self, expert, block):
        return policy_mode(self.handle, expert, block)

    def close(self):
        if self.handle is not None and _lib is not None:
            policy_destroy(self.handle)
        self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def qlinear_workspace_bytes(mode, M, K):
    out = ctypes.c_size_t()
    _check(lib().mxq_qlinear_workspace_bytes(int(mode), int(M), int(K), ctypes.byref(out)),
           "qlinear_workspace_bytes")
    return out.value


def qlinear(policy, expert, block, x, w_codes, w_scales, bias=None, epilogue=EPI_NONE,
            y=None, workspace=None, stream=None):
    """One quantized linear under the policy: quantize x with (expert, block)'s mode, then GEMM."""
    torch = _torch()
    handle = policy.handle if isinstance(policy, Policy) else policy
    m, k = _rows_k(x, "x")
    n = int(w_codes.shape[0])
    if y is None:
        y = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        mode = policy_mode(handle, expert, block)
        workspace = torch.empty((max(qlinear_workspace_bytes(mode, m, k), 1),), dtype=torch.uint8,
                                device=x.device)
    st = lib().mxq_qlinear(handle, int(expert), int(block), _dev_ptr(x, "x", torch.bfloat16), m, k,
                            _dev_ptr(w_codes, "w_codes", torch.uint8), _dev_ptr(w_scales, "w_scales", torch.uint8),
                            n, _dev_ptr(bias, "bias", torch.bfloat16), int(epilogue),
                            _dev_ptr(y, "y", torch.bfloat16), _dev_ptr(workspace, "workspace", torch.uint8),
                            int(workspace.numel()), _stream_handle(stream))
    _check(st, "qlinear")
    return y


def qlinear_noalloc(policy, expert, block, x, w_codes, w_scales, y, bias=None, epilogue=EPI_NONE, stream=None):
    """qlinear into a caller-provided y with the library's fixed scratch area instead of a workspace.

    Allocates nothing (y must be given); calls that overlap on one device race on the scratch area."""
    torch = _torch()
    handle = policy.handle if isinstance(policy, Policy) else policy
    m, k = _rows_k(x, "x")
    n = int(w_codes.shape[0])
    st = lib().mxq_qlinear_noalloc(handle, int(expert), int(block), _dev_ptr(x, "x", torch.bfloat16), m, k,
                                    _dev_ptr(w_codes, "w_codes", torch.uint8),
                                    _dev_ptr(w_scales, "w_scales", torch.uint8), n,
                                    _dev_ptr(bias, "bias", torch.bfloat16), int(epilogue),
                                    _dev_ptr(y, "y", torch.bfloat16), _stream_handle(stream))
    _check(st, "qlinear_noalloc")
    return y


def qlinear_transform(policy, expert, block, x, w_codes, w_scales, act_mult=None, bias=None, epilogue=EPI_NONE,
                      y=None, workspace=None, stream=None):
    """qlinear for tables with transform_on blocks: such a block quantizes x with its ``act_mult``."""
    torch = _torch()
    handle = policy.handle if isinstance(policy, Policy) else policy
    m, k = _rows_k(x, "x")
    n = int(w_codes.shape[0])
    if y is None:
        y = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        mode = policy_mode(handle, expert, block)
        workspace = torch.empty((max(qlinear_workspace_bytes(mode, m, k), 1),), dtype=torch.uint8,
                                device=x.device)
    st = lib().mxq_qlinear_transform(handle, int(expert), int(block), _dev_ptr(x, "x", torch.bfloat16), m, k,
                                      _dev_ptr(w_codes, "w_codes", torch.uint8),
                                      _dev_ptr(w_scales, "w_scales", torch.uint8), n,
                                      _dev_ptr(bias, "bias", torch.bfloat16), int(epilogue),
                                      _dev_ptr(act_mult, "act_mult", torch.float32),
                                      _dev_ptr(y, "y", torch.bfloat16), _dev_ptr(workspace, "workspace", torch.uint8),
                                      int(workspace.numel()), _stream_handle(stream))
    _check(st, "qlinear_transform")
    return y


# ----------------------------------------------------------- selection ----

def sqnr_accumulate(y, y_ref, sums, stream=None):
    """Fold bf16 y against bf16 y_ref (same size) into sums (device float64 [2]: signal, noise)."""
    torch = _torch()
    if y.numel() != y_ref.numel():
        raise ValueError("y and y_ref differ in size")
    st = lib().mxq_sqnr_accumulate(_dev_ptr(y, "y", torch.bfloat16), _dev_ptr(y_ref, "y_ref", torch.bfloat16),
                                    int(y.numel()), _dev_ptr(sums, "sums", torch.float64), _stream_handle(stream))
    _check(st, "sqnr_accumulate")
    return sums


def _replay_array(linears):
    torch = _torch()
    arr = (ReplayLinear * len(linears))()
    for i, (x, w, y_ref) in enumerate(linears):
        m, k = _rows_k(x, "x")
        n = int(w.shape[0])
        if tuple(w.shape) != (n, k) or tuple(y_ref.shape) != (m, n):
            raise ValueError("replay linear shapes must be x [M, K], w [N, K], y_ref [M, N]")
        arr[i] = ReplayLinear(_dev_ptr(x, "x", torch.bfloat16), _dev_ptr(w, "w", torch.bfloat16),
                              _dev_ptr(y_ref, "y_ref", torch.bfloat16), m, n, k)
    return arr


def replay_workspace_bytes(linears):
    arr = _replay_array(linears)
    out = ctypes.c_size_t()
    _check(lib().mxq_replay_workspace_bytes(arr, len(linears), ctypes.byref(out)), "replay_workspace_bytes")
    return out.value


def block_replay_sqnr(linears, sums_off, sums_on, workspace=None, stream=None):
    """Replay one block's linears [(x, w, y_ref), ...] OFF and ON, folding into sums_off / sums_on."""
    torch = _torch()
    arr = _replay_array(linears)
    if workspace is None:
        workspace = torch.empty((max(replay_workspace_bytes(linears), 1),), dtype=torch.uint8,
                                device=sums_off.device)
    st = lib().mxq_block_replay_sqnr(arr, len(linears), _dev_ptr(workspace, "workspace", torch.uint8),
                                      int(workspace.numel()), _dev_ptr(sums_off, "sums_off", torch.float64),
                                      _dev_ptr(sums_on, "sums_on", torch.float64), _stream_handle(stream))
    _check(st, "block_replay_sqnr")


def policy_select(sums_off, sums_on, tier=TIER_HIGH):
    """Host float64 [n_experts, n_blocks, 2] sums (OFF, ON) -> uint8 policy artifact [n_experts, n_blocks]."""
    off = np.ascontiguousarray(sums_off, np.float64)
    on = np.ascontiguousarray(sums_on, np.float64)
    if off.ndim != 3 or off.shape[2] != 2 or on.shape != off.shape:
        raise ValueError("sums must be float64 [n_experts, n_blocks, 2]")
    modes = np.empty(off.shape[:2], np.uint8)
    st = lib().mxq_policy_select(off.ctypes.data_as(_P), on.ctypes.data_as(_P), off.shape[0], off.shape[1],
                                  int(tier), modes.ctypes.data_as(_P))
    _check(st, "policy_select")
    return modes


# ------------------------------------------------------------ low rank ----

def lowrank_down(x, l1t, t=None, stream=None):
    """SVDQuant branch, first half: t [M, r] = bf16(x [M, K] @ L1), with L1 given transposed as l1t [r, K]."""
    torch = _torch()
    m, k = _rows_k(x, "x")
    r = int(l1t.shape[0])
    if t is None:
        t = torch.empty((m, r), dtype=torch.bfloat16, device=x.device)
    st = lib().mxq_lowrank_down(_dev_ptr(x, "x", torch.bfloat16), m, k, _dev_ptr(l1t, "l1t", torch.bfloat16), r,
                                 _dev_ptr(t, "t", torch.bfloat16), _stream_handle(stream))
    _check(st, "lowrank_down")
    return t


def gemm_lowrank(a_codes, a_scales, w_codes, w_scales, t, l2, bias=None, epilogue=EPI_NONE, y=None, y_scales=None,
                 mxfp4_out=False, stream=None):
    """W4A4 GEMM with SVDQuant's branch t @ l2^T in its fp32 sums, rounded to bf16 once.

    bf16 output y [M, N] by default; with ``mxfp4_out`` (or y_scales given) the output is the
    next W4A4 layer's activation, (y_codes, y_scales), as gemm_mxfp4_out writes it."""
    torch = _torch()
    m = int(a_codes.shape[0])
    n = int(w_codes.shape[0])
    k = int(w_codes.shape[1]) * 2
    r = int(t.shape[1])
    if tuple(t.shape) != (m, r) or tuple(l2.shape) != (n, r):
        raise ValueError(f"t must be [{m}, r] and l2 [{n}, r]; got {tuple(t.shape)} and {tuple(l2.shape)}")
    mxfp4_out = mxfp4_out or y_scales is not None
    if mxfp4_out and (y is None or y_scales is None):
        y, y_scales = act_buffers(W4A4, m, n, w_codes.device)
    elif y is None:
        y = torch.empty((m, n), dtype=torch.bfloat16, device=w_codes.device)
    st = lib().mxq_gemm_lowrank(_dev_ptr(a_codes, "a_codes"), _dev_ptr(a_scales, "a_scales"),
                                 _dev_ptr(w_codes, "w_codes", torch.uint8), _dev_ptr(w_scales, "w_scales", torch.uint8),
                                 _dev_ptr(bias, "bias", torch.bfloat16), _dev_ptr(t, "t", torch.bfloat16),
                                 _dev_ptr(l2, "l2", torch.bfloat16), r, int(epilogue),
                                 _dev_ptr(y, "y", torch.uint8 if mxfp4_out else torch.bfloat16),
                                 _dev_ptr(y_scales, "y_scales", torch.uint8), m, n, k, _stream_handle(stream))
    _check(st, "gemm_lowrank")
    return (y, y_scales) if mxfp4_out else y


def gemm_lowrank_supported(M, N, K, mxfp4_out=False):
    """Whether gemm_lowrank takes (M, N, K): the pipelined kernel's shapes (for MXFP4 output N % 128 == 0
    and the output below 2 GiB)."""
    return gemm_kernel_name(W4A4, M, N, K).startswith("pipe_") and (
        not mxfp4_out or (N % 128 == 0 and M * (N // 2) < 2 ** 31 - 256))


def quantize_act_lowrank(x, l1t, codes=None, scales=None, t=None, stream=None):
    """W4A4 activation codes/scales of x and the branch's t = bf16(x @ L1) in one pass over x.

    Same bytes as quantize_act(W4A4, x) and the same t as lowrank_down(x, l1t). Returns
    (codes, scales, t)."""
    torch = _torch()
    m, k = _rows_k(x, "x")
    r = int(l1t.shape[0])
    if tuple(l1t.shape) != (r, k):
        raise ValueError(f"l1t must be [r, {k}], got {tuple(l1t.shape)}")
    if codes is None or scales is None:
        codes, scales = act_buffers(W4A4, m, k, x.device)
    if t is None:
        t = torch.empty((m, r), dtype=torch.bfloat16, device=x.device)
    if tuple(t.shape) != (m, r):
        raise ValueError(f"t must be [{m}, {r}], got {tuple(t.shape)}")
    st = lib().mxq_quantize_act_lowrank(_dev_ptr(x, "x", torch.bfloat16), m, k, _dev_ptr(l1t, "l1t", torch.bfloat16), r,
                                         _dev_ptr(codes, "codes", torch.uint8), _dev_ptr(scales, "scales", torch.uint8),
                                         _dev_ptr(t, "t", torch.bfloat16), _stream_handle(stream))
    _check(st, "quantize_act_lowrank")
    return codes, scales, t


def lowrank_up(y_pre, t, l2, epilogue=EPI_NONE, y=None, stream=None):
    """SVDQuant branch, second half: y = bf16(epilogue(y_pre + t @ l2^T)); l2 [N, r]; y may be y_pre."""
    torch = _torch()
    m, n = _rows_k(y_pre, "y_pre")
    r = int(t.shape[1])
    if y is None:
        y = torch.empty_like(y_pre)
    st = lib().mxq_lowrank_up(_dev_ptr(y_pre, "y_pre", torch.bfloat16), _dev_ptr(t, "t", torch.bfloat16),
                               _dev_ptr(l2, "l2", torch.bfloat16), m, n, r, int(epilogue),
                               _dev_ptr(y, "y", torch.bfloat16), _stream_handle(stream))
    _check(st, "lowrank_up")
    return y
