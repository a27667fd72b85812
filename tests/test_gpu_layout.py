"""GPU tests of the canonical-layout conversions (mxq_mxfp4_to_canonical,
mxq_mxfp4_from_canonical): the OCP MXFP4 layout is row-major codes
[rows][K/2] (element 2t in the low nibble of byte t) and scales [rows][K/32],
which is exactly what the oracle's quantizer returns.

* exported weight and activation codes and scales equal the oracle's byte
  for byte (ragged K included, where the last code panel is narrower);
* import(export(x)) gives back the library buffers byte for byte, the zero
  padding of the last scale group included;
* weights held in the OCP layout (the oracle's own packing) go through
  import into mxq_gemm and give the same output, bit for bit, as the
  library's own packing, and the oracle's result within the tolerance.
"""

import sys

import numpy as np
import pytest
import torch

import mx_bit_quantized_amd as mxq
import oracle
import synth
from gpu_util import assert_codes_equal, assert_output_close, dev_bf16, host_bits, host_u8

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


def _u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).to("cuda:0")


def _edge_rows(m, k, seed):
    g = np.random.default_rng(seed)
    x = synth.activation_bf16(seed, m, k, ("student_t",))
    x[0] = 0
    x[1] = (g.integers(0, 0x80, k) | (g.integers(0, 2, k) << 15)).astype(np.uint16)  # subnormals
    x[2, k - 1] = 0x8000
    x[3] = synth.f32_to_bf16_bits((g.standard_normal(k) * 1e30).astype(np.float32))
    return x


@pytest.mark.parametrize("rows,k", [(300, 512), (40, 96), (37, 160), (129, 1056), (64, 5120), (1, 32)])
def test_export_equals_oracle_layout(rows, k):
    say("export", rows, k)
    w = synth.weight_bf16(rows + k, rows, k)
    x = _edge_rows(max(rows, 4), k, rows * 3 + k)
    for what, bits, pack in (("weight", w, lambda t: mxq.quantize_weight_mxfp4(t)),
                             ("activation", x, lambda t: mxq.quantize_act(mxq.W4A4, t))):
        n = bits.shape[0]
        codes, scales = pack(dev_bf16(bits))
        c_rm, s_rm = mxq.mxfp4_to_canonical(codes, scales, n, k)
        torch.cuda.synchronize()
        want_c, want_s = oracle.mxfp4_quantize(bits)
        assert_codes_equal(host_u8(c_rm), want_c, f"{what} canonical codes [{n}x{k}]")
        assert_codes_equal(host_u8(s_rm), want_s, f"{what} canonical scales [{n}x{k}]")


@pytest.mark.parametrize("rows,k", [(300, 512), (40, 96), (37, 160), (129, 1056), (257, 5120)])
def test_import_of_export_is_identity(rows, k):
    say("round trip", rows, k)
    x = _edge_rows(rows, k, 11 * rows + k)
    codes, scales = mxq.quantize_act(mxq.W4A4, dev_bf16(x))
    c_rm, s_rm = mxq.mxfp4_to_canonical(codes, scales, rows, k)
    # fill the destinations with junk first: every byte must be written
    c2 = torch.full_like(codes, 0xA5)
    s2 = torch.full_like(scales, 0x5A)
    mxq.mxfp4_from_canonical(c_rm, s_rm, c2, s2)
    torch.cuda.synchronize()
    assert torch.equal(c2, codes), "codes differ after import(export)"
    assert torch.equal(s2, scales), "scales (or their zero padding) differ after import(export)"


@pytest.mark.parametrize("mode", [mxq.W4A4, mxq.W4A8])
@pytest.mark.parametrize("m,n,k", [(300, 512, 640), (64, 200, 160), (1000, 1280, 896)])
def test_gemm_on_imported_ocp_weights(mode, m, n, k):
    say("gemm on imported weights", mode, m, n, k)
    w = synth.weight_bf16(m + n, n, k)
    x = synth.activation_bf16(m + k, m, k, ("student_t",))
    owc, ows = oracle.mxfp4_quantize(w)                     # OCP row-major, from the oracle
    wc, ws = mxq.mxfp4_from_canonical(_u8(owc), _u8(ows))   # into the library layout
    wc_lib, ws_lib = mxq.quantize_weight_mxfp4(dev_bf16(w))
    torch.cuda.synchronize()
    assert torch.equal(wc, wc_lib) and torch.equal(ws, ws_lib), "imported weights differ from the library's packing"
    ac, asc = mxq.quantize_act(mode, dev_bf16(x))
    y = host_bits(mxq.gemm(mode, ac, asc, wc, ws))
    oac, oas = oracle.quantize_act(mode, x)
    assert_output_close(y, oracle.qdq_matmul(mode, oac, oas, owc, ows), f"gemm on imported weights mode={mode}")


def test_fused_mxfp4_output_exports_like_the_quantizer():
    """mxq_gemm_mxfp4_out's output in OCP layout equals the library quantizer's on the GEMM's bf16 output.

    (That the fused codes equal the oracle's is tested against the oracle's own
    bf16 rounding in test_gpu_fused.py; here only the export of a GEMM-written
    buffer is at stake, so both sides come from the library and the layout is
    also undone on the host, independently of the export.)"""
    from gpu_util import code_rows, group_major_scales
    m, n, k = 600, 1024, 512
    say("fused export", m, n, k)
    x = synth.activation_bf16(21, m, k, ("student_t",))
    w = synth.weight_bf16(22, n, k)
    wc, ws = mxq.quantize_weight_mxfp4(dev_bf16(w))
    ac, asc = mxq.quantize_act(mxq.W4A4, dev_bf16(x))
    assert mxq.gemm_mxfp4_out_supported(m, n, k)
    hc, hs = mxq.gemm_mxfp4_out(ac, asc, wc, ws, None, mxq.EPI_GELU_TANH)
    qc, qs = mxq.quantize_act(mxq.W4A4, mxq.gemm(mxq.W4A4, ac, asc, wc, ws, None, mxq.EPI_GELU_TANH))
    c_rm, s_rm = mxq.mxfp4_to_canonical(hc, hs, m, n)
    q_rm, qs_rm = mxq.mxfp4_to_canonical(qc, qs, m, n)
    torch.cuda.synchronize()
    assert torch.equal(c_rm, q_rm) and torch.equal(s_rm, qs_rm), "fused output exports differently"
    assert_codes_equal(host_u8(c_rm), code_rows(hc, m, n, 4), "export vs host-side panel order")
    assert_codes_equal(group_major_scales(host_u8(s_rm)), host_u8(hs), "export vs host-side scale order")
