"""ctypes access to libmxq_hostcheck.so: the kernels' element conversions built
for the CPU (see mx_bit_quantized_amd/csrc/mxq_hostcheck.cpp)."""

import ctypes
import os

import numpy as np

from conftest import ROOT

PATH = os.path.join(ROOT, "mx_bit_quantized_amd", "libmxq_hostcheck.so")
_P = ctypes.c_void_p
_I64 = ctypes.c_int64

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(PATH):
            raise RuntimeError(f"{PATH} missing: run `python -m mx_bit_quantized_amd._build`")
        l = ctypes.CDLL(PATH)
        l.mxq_host_mx_scale_bytes.argtypes = [_P, _I64, _P]
        l.mxq_host_e2m1_codes.argtypes = [_P, _I64, ctypes.c_uint32, _P]
        l.mxq_host_e4m3fn_codes.argtypes = [_P, _I64, _P]
        l.mxq_host_mxfp4_quantize.argtypes = [_P, _I64, _I64, _P, _P]
        l.mxq_host_fp8_quantize.argtypes = [_P, _I64, _I64, _P, _P]
        l.mxq_host_fp8_division_sweep.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(_I64),
                                                  ctypes.POINTER(_I64), ctypes.POINTER(_I64)]
        l.mxq_host_fp8_static_sweep.argtypes = [_P, _I64, ctypes.POINTER(_I64), ctypes.POINTER(_I64),
                                                ctypes.POINTER(_I64)]
        l.mxq_host_fp8_quantize_static.argtypes = [_P, _I64, _I64, ctypes.c_float, _P, _P]
        l.mxq_host_bf16_rne.argtypes = [_P, _I64, _P]
        l.mxq_host_gelu_tanh.argtypes = [_P, _I64, _P]
        _lib = l
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def scale_bytes(amax_bits):
    a = np.ascontiguousarray(amax_bits, np.uint16)
    out = np.empty(a.shape, np.uint8)
    lib().mxq_host_mx_scale_bytes(_p(a), a.size, _p(out))
    return out


def e2m1_codes(bits, scale_byte):
    a = np.ascontiguousarray(bits, np.uint16)
    out = np.empty(a.shape, np.uint8)
    lib().mxq_host_e2m1_codes(_p(a), a.size, int(scale_byte), _p(out))
    return out


def e4m3fn_codes(q):
    a = np.ascontiguousarray(q, np.float32)
    out = np.empty(a.shape, np.uint8)
    lib().mxq_host_e4m3fn_codes(_p(a), a.size, _p(out))
    return out


def mxfp4_quantize(x_bits):
    x = np.ascontiguousarray(x_bits, np.uint16)
    r, k = x.shape
    codes = np.empty((r, k // 2), np.uint8)
    scales = np.empty((r, k // 32), np.uint8)
    lib().mxq_host_mxfp4_quantize(_p(x), r, k, _p(codes), _p(scales))
    return codes, scales


def fp8_quantize(x_bits):
    x = np.ascontiguousarray(x_bits, np.uint16)
    r, k = x.shape
    codes = np.empty((r, k), np.uint8)
    scales = np.empty((r,), np.float32)
    lib().mxq_host_fp8_quantize(_p(x), r, k, _p(codes), _p(scales))
    return codes, scales


def fp8_division_sweep(lo, hi):
    a, b, c = _I64(), _I64(), _I64()
    lib().mxq_host_fp8_division_sweep(int(lo), int(hi), ctypes.byref(a), ctypes.byref(b), ctypes.byref(c))
    return a.value, b.value, c.value


def bf16_rne(f):
    a = np.ascontiguousarray(f, np.float32)
    out = np.empty(a.shape, np.uint16)
    lib().mxq_host_bf16_rne(_p(a), a.size, _p(out))
    return out


def gelu_tanh(f):
    a = np.ascontiguousarray(f, np.float32)
    out = np.empty(a.shape, np.float32)
    lib().mxq_host_gelu_tanh(_p(a), a.size, _p(out))
    return out


def fp8_static_sweep(amax):
    a = np.ascontiguousarray(amax, np.float32)
    pairs, qm, cm = _I64(), _I64(), _I64()
    lib().mxq_host_fp8_static_sweep(_p(a), a.size, ctypes.byref(pairs), ctypes.byref(qm), ctypes.byref(cm))
    return pairs.value, qm.value, cm.value


def fp8_quantize_static(x_bits, amax):
    x = np.ascontiguousarray(x_bits, np.uint16)
    r, k = x.shape
    codes = np.empty((r, k), np.uint8)
    scales = np.empty((r,), np.float32)
    lib().mxq_host_fp8_quantize_static(_p(x), r, k, float(amax), _p(codes), _p(scales))
    return codes, scales
