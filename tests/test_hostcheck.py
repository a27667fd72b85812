"""The kernels' element conversions, built for the CPU, against the oracle
over every bf16 input (CPU only). A mismatch here would be a bit-exactness
failure on the GPU too, found before any GPU run."""

from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np
import pytest
import torch

import oracle
import synth
import hostcheck


def finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    return bits[((bits >> 7) & 0xFF) != 0xFF]


def test_scale_byte_all_bf16_magnitudes():
    bits = finite_bf16()
    got = hostcheck.scale_bytes(bits)
    want = oracle.mxfp4_scale_exponent(np.abs(oracle.bf16_bits_to_f64(bits))) + 127
    assert np.array_equal(got.astype(np.int64), want)


def test_e2m1_codes_every_bf16_times_every_scale():
    bits = finite_bf16()
    v = oracle.bf16_bits_to_f64(bits)
    for sb in range(0, 253):
        got = hostcheck.e2m1_codes(bits, sb)
        want = oracle.e2m1_encode(v / np.ldexp(1.0, sb - 127))
        # only elements that can share a block with scale byte sb matter
        # (|v| < 8 * 2^E); larger ones would have raised the block's scale
        live = np.abs(v) < 8.0 * np.ldexp(1.0, sb - 127)
        bad = np.nonzero((got != want) & live)[0]
        assert bad.size == 0, (sb, [hex(int(bits[i])) for i in bad[:5]], got[bad[:5]], want[bad[:5]])


def test_e4m3fn_codes_dense_fp32_set():
    g = np.random.default_rng(0)
    mids = (oracle.e4m3fn_decode(np.arange(0x7E, dtype=np.uint8))
            + oracle.e4m3fn_decode(np.arange(1, 0x7F, dtype=np.uint8))) / 2
    mids32 = mids.astype(np.float32)
    q = np.concatenate([
        oracle.bf16_bits_to_f32(finite_bf16()),
        mids32, np.nextafter(mids32, np.float32(np.inf)), np.nextafter(mids32, np.float32(0)),
        g.uniform(-448, 448, 200000).astype(np.float32),
        (np.ldexp(g.uniform(1, 2, 200000), g.integers(-160, 9, 200000)) * g.choice([-1, 1], 200000)).astype(np.float32),
        np.array([448.0, 463.99, 464.0, 448.0001, -448.0001, 2.0 ** -10, 2.0 ** -149, -0.0], np.float32),
    ])
    q = q[np.abs(q) < 464.0]  # the kernel's quotients never reach 464
    got = hostcheck.e4m3fn_codes(q)
    want = oracle.e4m3fn_encode(q.astype(np.float64))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (q[bad[:5]], got[bad[:5]], want[bad[:5]])


@pytest.mark.slow
def test_fp8_quotient_equals_ieee_division_every_bf16_pair():
    """Every positive finite bf16 amax, every bf16 x with |x| <= amax, both signs."""
    edges = np.linspace(1, 0x7F80, 65).astype(int)
    # later ranges hold more pairs; interleave chunk sizes across the pool
    chunks = list(zip(edges[:-1], edges[1:]))
    workers = min(8, os.cpu_count() or 1)
    with ThreadPoolExecutor(workers) as ex:
        res = list(ex.map(lambda c: hostcheck.fp8_division_sweep(*c), chunks))
    pairs = sum(r[0] for r in res)
    assert pairs > 1_000_000_000
    assert sum(r[1] for r in res) == 0, "quotient differs from IEEE x / s"
    assert sum(r[2] for r in res) == 0, "E4M3FN code differs"


def test_fp8_quotient_sampled_pairs():
    """A quick slice of the exhaustive sweep for the default CPU run."""
    for lo in (1, 0x0080, 0x1F00, 0x2D00, 0x3F00, 0x4300, 0x7E00):
        pairs, qm, cm = hostcheck.fp8_division_sweep(lo, lo + 24)
        assert pairs > 0 and qm == 0 and cm == 0, (hex(lo), qm, cm)


def _edge_rows(k):
    g = np.random.default_rng(42)
    rows = [
        synth.activation_bf16(7, 24, k, ("student_t",)),
        synth.activation_bf16(7, 8, k, ("scaled", 4, 20.0)),
        np.zeros((2, k), np.uint16),
        (g.integers(0, 0x0080, (3, k)) | (g.integers(0, 2, (3, k)) << 15)).astype(np.uint16),  # subnormal
        synth.f32_to_bf16_bits(g.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], (4, k)).astype(np.float32)
                               * g.choice([-1, 1], (4, k)).astype(np.float32)),  # FP4 ties
        synth.f32_to_bf16_bits((g.standard_normal((3, k)) * 1e30).astype(np.float32)),
        np.full((1, k), 0x7F7F, np.uint16),  # largest finite bf16
    ]
    x = np.concatenate(rows)
    x[2, 5] = 0x8000  # a -0 in a zero row
    return x


@pytest.mark.parametrize("k", [32, 96, 512])
def test_mxfp4_row_composition_matches_oracle(k):
    x = _edge_rows(k)
    got = hostcheck.mxfp4_quantize(x)
    want = oracle.mxfp4_quantize(x)
    assert np.array_equal(got[1], want[1])
    assert np.array_equal(got[0], want[0])


@pytest.mark.parametrize("k", [32, 96, 512])
def test_fp8_row_composition_matches_oracle(k):
    x = _edge_rows(k)
    got = hostcheck.fp8_quantize(x)
    want = oracle.fp8_quantize_per_token(x)
    assert np.array_equal(got[1].view(np.uint32), want[1].view(np.uint32))
    assert np.array_equal(got[0], want[0])


def test_bf16_rne_matches_torch():
    g = np.random.default_rng(1)
    f = np.concatenate([g.standard_normal(100000).astype(np.float32) * 1e3,
                        (np.arange(1 << 16, dtype=np.uint32) << 16 | 0x8000).view(np.float32)])
    f = f[np.isfinite(f)]
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(hostcheck.bf16_rne(f), want)


def test_gelu_tanh_fp32_close_to_oracle():
    y = np.linspace(-20, 20, 100001).astype(np.float32)
    got = hostcheck.gelu_tanh(y).astype(np.float64)
    want = oracle.gelu_tanh(y.astype(np.float64))
    assert np.all(np.abs(got - want) <= 4e-7 * np.abs(want) + 1e-7)


def _static_amax_set():
    g = np.random.default_rng(77)
    vals = [np.float32(v) for v in (448.0, 224.0, 1.0, 3.296875, 0.0, 1e-44, 1e-40, 2.4e-17, 2.43e-17, 1e-30,
                                     3.3895314e38, 3.0e38, 65504.0, 5.27e-36)]
    rnd = np.ldexp(g.uniform(1, 2, 160), g.integers(-149, 127, 160)).astype(np.float32)
    pow2 = np.ldexp(1.0, np.arange(-140, 127, 9)).astype(np.float32)
    a = np.concatenate([np.array(vals, np.float32), rnd, pow2])
    return a[np.isfinite(a)]


def test_fp8_static_quotient_and_code_sweep():
    """Static scales (any fp32 amax, subnormal and huge ones too) against every finite bf16 x:
    the kernel's clamped quotient and code equal IEEE division followed by saturating RNE."""
    amax = _static_amax_set()
    chunks = np.array_split(amax, 8)
    with ThreadPoolExecutor(8) as ex:
        res = list(ex.map(hostcheck.fp8_static_sweep, chunks))
    pairs = sum(r[0] for r in res)
    assert pairs == len(amax) * 0x7F80 * 2
    assert sum(r[1] for r in res) == 0, "quotient differs from IEEE x / s"
    assert sum(r[2] for r in res) == 0, "E4M3FN code differs"


@pytest.mark.parametrize("k", [32, 96, 512])
def test_fp8_static_composition_matches_oracle(k):
    x = _edge_rows(k)
    true_amax = float(np.abs(oracle.bf16_bits_to_f64(x)).max())
    for amax in (true_amax, true_amax * 1e-3, 0.0, 1e-42, 3.0e38):
        got = hostcheck.fp8_quantize_static(x, np.float32(amax))
        want = oracle.fp8_quantize_static(x, np.float32(amax))
        assert np.array_equal(got[1].view(np.uint32), want[1].view(np.uint32)), amax
        assert np.array_equal(got[0], want[0]), amax
