// mxq_hostcheck.cpp - host build of the kernels' element conversions.
//
// libmxq_hostcheck.so exposes the __host__ __device__ functions of
// mxq_convert.h, compiled for the CPU, so that the CPU test suite can compare
// the exact arithmetic the gfx950 kernels run against the oracle over every
// bf16 input, without a GPU. It also mirrors the per-block / per-row
// composition of the quantizer kernels (block amax over magnitude bits, scale
// byte, nibble packing, per-row FP8 setup). Not used by the product path.
#include <math.h>
#include <stdint.h>

#include "mxq_convert.h"

using namespace mxq;

extern "C" {

// Scale bytes for block amax magnitude bit patterns.
void mxq_host_mx_scale_bytes(const uint16_t* amax_bits, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)mx_scale_byte(amax_bits[i] & 0x7FFFu);
}

// 4-bit codes of bf16 values quantized against one scale byte.
void mxq_host_e2m1_codes(const uint16_t* bits, int64_t n, uint32_t scale_byte, uint8_t* out) {
  const float inv = mx_inv_scale(scale_byte);
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)e2m1_code_bf16(bits[i], inv);
}

// E4M3FN codes of fp32 values.
void mxq_host_e4m3fn_codes(const float* q, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)e4m3fn_code(q[i]);
}

// The quantizer kernels' composition, row by row (dense rows, ld = K).
void mxq_host_mxfp4_quantize(const uint16_t* x, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales) {
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < K / 32; ++b) {
      const uint16_t* v = x + r * K + b * 32;
      uint32_t amax = 0;
      for (int i = 0; i < 32; ++i) amax = umax(amax, v[i] & 0x7FFFu);
      const uint32_t sb = mx_scale_byte(amax);
      const float inv = mx_inv_scale(sb);
      for (int i = 0; i < 16; ++i) {
        uint32_t lo = e2m1_code_bf16(v[2 * i], inv);
        uint32_t hi = e2m1_code_bf16(v[2 * i + 1], inv);
        codes[r * (K / 2) + b * 16 + i] = (uint8_t)(lo | (hi << 4));
      }
      scales[r * (K / 32) + b] = (uint8_t)sb;
    }
  }
}

void mxq_host_fp8_quantize(const uint16_t* x, int64_t rows, int64_t K, uint8_t* codes, float* scales) {
  for (int64_t r = 0; r < rows; ++r) {
    const uint16_t* v = x + r * K;
    uint32_t amax = 0;
    for (int64_t i = 0; i < K; ++i) amax = umax(amax, v[i] & 0x7FFFu);
    const Fp8Row row = fp8_row_setup(amax);
    for (int64_t i = 0; i < K; ++i) codes[r * K + i] = (uint8_t)fp8_code_bf16(v[i], row);
    scales[r] = row.s;
  }
}

// For every positive finite bf16 amax pattern in [amax_lo, amax_hi) and every
// bf16 x with |x| <= amax (both signs): compare the kernel quotient against
// the IEEE fp32 quotient x / s. Counts pairs, quotient mismatches among
// quotients of magnitude >= 2^-10 (smaller ones can only give a zero code),
// and final E4M3FN code mismatches.
void mxq_host_fp8_division_sweep(int32_t amax_lo, int32_t amax_hi, int64_t* pairs,
                                 int64_t* quotient_mismatch, int64_t* code_mismatch) {
  int64_t np = 0, nq = 0, nc = 0;
  for (int32_t a = amax_lo; a < amax_hi; ++a) {
    if (a <= 0 || a >= 0x7F80) continue;
    const Fp8Row row = fp8_row_setup((uint32_t)a);
    for (int32_t m = 0; m <= a; ++m) {
      for (int sgn = 0; sgn < 2; ++sgn) {
        const uint32_t bits = (uint32_t)m | (sgn ? 0x8000u : 0u);
        const float x = as_float(bits << 16);
        const float ref = x / row.s;
        const float got = fp8_quotient(x, row);
        ++np;
        if (fabsf(ref) >= 0.0009765625f && as_uint(ref) != as_uint(got)) ++nq;
        if (e4m3fn_code(ref) != fp8_code_bf16(bits, row)) ++nc;
      }
    }
  }
  *pairs = np;
  *quotient_mismatch = nq;
  *code_mismatch = nc;
}

// Static scales: for each fp32 amax in the list and every finite bf16 x (both
// signs), compare the kernel code with the saturating E4M3FN code of the IEEE
// quotient x / s (infinite quotients included), and the kernel quotient with
// the IEEE one wherever |x / s| lies in [2^-10, 448].
void mxq_host_fp8_static_sweep(const float* amax, int64_t n_amax, int64_t* pairs, int64_t* quotient_mismatch,
                               int64_t* code_mismatch) {
  int64_t np = 0, nq = 0, nc = 0;
  for (int64_t i = 0; i < n_amax; ++i) {
    const Fp8Row row = fp8_scale_setup(amax[i]);
    for (uint32_t m = 0; m < 0x7F80u; ++m) {
      for (int sgn = 0; sgn < 2; ++sgn) {
        const uint32_t bits = m | (sgn ? 0x8000u : 0u);
        const float x = as_float(bits << 16);
        const uint32_t sign = sgn ? 0x80u : 0u;
        uint32_t want;
        if (row.s == 0.0f) {
          want = sign;
        } else {
          const float ref = fabsf(x) / row.s;
          want = e4m3fn_code(ref) | sign;
          if (ref >= 0.0009765625f && ref <= 448.0f &&
              as_uint(ref) != as_uint(fp8_static_quotient(fabsf(x), row)))
            ++nq;
        }
        ++np;
        if (want != fp8_static_code_bf16(bits, row)) ++nc;
      }
    }
  }
  *pairs = np;
  *quotient_mismatch = nq;
  *code_mismatch = nc;
}

void mxq_host_fp8_quantize_static(const uint16_t* x, int64_t rows, int64_t K, float amax, uint8_t* codes,
                                  float* scales) {
  const Fp8Row row = fp8_scale_setup(amax);
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t i = 0; i < K; ++i) codes[r * K + i] = (uint8_t)fp8_static_code_bf16(x[r * K + i], row);
    scales[r] = row.s;
  }
}

void mxq_host_bf16_rne(const float* f, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint16_t)bf16_rne(f[i]);
}

void mxq_host_gelu_tanh(const float* f, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = gelu_tanh(f[i]);
}

}  // extern "C"
