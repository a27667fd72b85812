// mxq_convert.h - element conversions shared by the gfx950 kernels.
//
// Every function here is __host__ __device__: the kernels use them on the
// GPU, and a host build of the same code is checked exhaustively on the CPU
// (all bf16 inputs against the rounding rules) before it runs on a GPU.
//
// Formats: MXFP4 = E2M1 elements with one E8M0 scale per 32 along K, FP8 =
// E4M3FN (section "Quantization formats" of the page "Quark Mixed-Precision
// Quantization for Wan2.2 Video Generation on AMD Instinct GPUs"; bit layouts
// of the OCP MX v1.0 and OCP FP8 definitions).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MXQ_HD __host__ __device__ __forceinline__

namespace mxq {

MXQ_HD float as_float(uint32_t u) {
  union { uint32_t u; float f; } c;
  c.u = u;
  return c.f;
}

MXQ_HD uint32_t as_uint(float f) {
  union { uint32_t u; float f; } c;
  c.f = f;
  return c.u;
}

MXQ_HD uint32_t umin(uint32_t a, uint32_t b) { return a < b ? a : b; }
MXQ_HD uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// ---------------------------------------------------------------- MXFP4 ---

// E8M0 scale byte of a 32-element block from the largest magnitude bit
// pattern (bf16 bits with the sign cleared) in the block.
//   E = floor(log2 amax) - 2, clamped to [-127, 127]; byte = E + 127.
// For a normal bf16 the biased exponent field f gives floor(log2) = f - 127,
// so byte = f - 2. Zero and subnormal blocks (and f = 1, 2) clamp to byte 0
// (E = -127); the largest finite bf16 (f = 254) gives byte 252.
MXQ_HD uint32_t mx_scale_byte(uint32_t amax_mag_bits) {
  int f = (int)(amax_mag_bits >> 7);
  int b = f - 2;
  return b < 0 ? 0u : (uint32_t)b;
}

// 2^-E as an fp32 for a scale byte b (E = b - 127). b is at most 252 for a
// finite block, so 2^-E lies in [2^-125, 2^127]: always a normal float.
MXQ_HD float mx_inv_scale(uint32_t b) { return as_float((254u - b) << 23); }

// E2M1 magnitude code (0..7) of r = |v| / 2^E >= 0, which is below 8 for any
// element of its block. Round half to even, saturating at 6 (code 7).
//   r < 1  : the subnormal step 0.5 -> round(2r) gives 0, 1 or 2 (2 = 1.0).
//   r >= 1 : keep one mantissa bit of the fp32 r with round-half-even on the
//            22 dropped bits; the carry moves into the exponent naturally.
//            The fp32 biased exponent 127+e maps to FP4 exponent field e+1,
//            hence code = (bits >> 22) - 252.
MXQ_HD uint32_t e2m1_mag_code(float r) {
  uint32_t rb = as_uint(r);
  uint32_t sub = (uint32_t)__builtin_rintf(r * 2.0f);
  uint32_t t = rb + 0x1FFFFFu + ((rb >> 22) & 1u);
  uint32_t nor = umin((t >> 22) - 252u, 7u);
  return rb < 0x3F800000u ? sub : nor;
}

// Full 4-bit E2M1 code of a bf16 element (uint16 bits) in a block whose
// 2^-E is `inv_scale`. v * 2^-E is exact in fp32 (a power-of-two product of
// a bf16 value; results below 2^-126 may be subnormal, fp32 denormals are
// kept, and they round to 0 anyway).
MXQ_HD uint32_t e2m1_code_bf16(uint32_t bits16, float inv_scale) {
  float mag = as_float((bits16 & 0x7FFFu) << 16);
  uint32_t c = e2m1_mag_code(mag * inv_scale);
  return c | ((bits16 >> 12) & 8u);
}

// --------------------------------------------------------------- E4M3FN ---

// E4M3FN code of an fp32 value, round half to even, saturating at 448
// (0x7E), sign kept. Finite inputs only.
//   |q| < 2^-6 : subnormal E4M3 with step 2^-9. Adding 2^14 (whose fp32 ulp
//                is 2^-9) rounds |q| to that step with the fp32 adder's
//                round-half-even; the integer difference of the bit patterns
//                is the code (8 = 2^-6 carries into the first normal).
//   otherwise  : keep three mantissa bits with round-half-even on the 20
//                dropped bits; fp32 biased exponent 120+e' maps to E4M3
//                field e', hence code = (bits >> 20) - (120 << 3).
MXQ_HD uint32_t e4m3fn_code(float q) {
  uint32_t b = as_uint(q);
  uint32_t sign = (b >> 24) & 0x80u;
  uint32_t a = b & 0x7FFFFFFFu;
  uint32_t sub = as_uint(as_float(a) + 16384.0f) - 0x46800000u;
  uint32_t t = a + 0x7FFFFu + ((a >> 20) & 1u);
  uint32_t nor = (t >> 20) - (120u << 3);
  uint32_t c = a < 0x3C800000u ? sub : nor;
  return umin(c, 0x7Eu) | sign;
}

// Per-row FP8 division setup. The quotient x / s must be the IEEE fp32
// quotient. With y = RN(1/s) (one IEEE division per row), each element uses
//   q0 = RN(x * y);  r = fma(-q0, s, x) (exact);  q = RN(q0 + r * y)
// which returns RN(x / s) when y is the correctly rounded reciprocal and the
// residual r is exact (Markstein's correction step). r is exact when its
// quantum 2^(e(x) - 46) is at least fp32's 2^-149; for quotients that can
// reach a nonzero E4M3 code (|q| >= 2^-10) that holds once s >= 2^-64. Rows
// with a smaller scale (bf16 amax below about 2^-55) are first multiplied by
// 2^64, exact for both x and s, which leaves the quotient, and so its
// rounding, unchanged. The host build of this code is compared with IEEE
// division for every bf16 amax and every bf16 x of its row.
struct Fp8Row {
  float s;       // the stored scale fp32(amax) / 448
  float pre;     // 1, or 2^64 when s < 2^-64
  float ss;      // s * pre
  float y;       // RN(1 / ss)
  float hi;      // RN(448 ss): the static quotient's clamp (see below)
};

// Setup from an fp32 amax: a row's bf16 amax (exact in fp32) for per-token
// scales, or a calibrated amax for a static one.
MXQ_HD Fp8Row fp8_scale_setup(float amax) {
  Fp8Row r;
  r.s = amax / 448.0f;
  r.pre = r.s < 5.42101086242752217e-20f ? 18446744073709551616.0f : 1.0f;  // 2^-64, 2^64
  r.ss = r.s * r.pre;
  r.y = 1.0f / r.ss;
  r.hi = 448.0f * r.ss;
  return r;
}

MXQ_HD Fp8Row fp8_row_setup(uint32_t amax_mag_bits) { return fp8_scale_setup(as_float(amax_mag_bits << 16)); }

MXQ_HD float fp8_quotient(float x, const Fp8Row& r) {
  float xs = x * r.pre;
  float q0 = xs * r.y;
  float rem = __builtin_fmaf(-q0, r.ss, xs);
  return __builtin_fmaf(rem, r.y, q0);
}

// E4M3FN code of a bf16 element of a row (s == 0 gives a signed zero code).
// Rounding to nearest is symmetric and s > 0, so the quotient is formed from
// |x| and x's sign bit is attached to the code; this also keeps -0 (the FMA
// correction would turn -0 into +0).
MXQ_HD uint32_t fp8_code_bf16(uint32_t bits16, const Fp8Row& r) {
  const uint32_t sign = (bits16 >> 8) & 0x80u;
  if (r.s == 0.0f) return sign;
  return e4m3fn_code(fp8_quotient(as_float((bits16 & 0x7FFFu) << 16), r)) | sign;
}

// Static (per-tensor) scale: x may exceed the calibrated amax, and quotients
// beyond 448 saturate. The pre-scaled |x| is first clamped at hi = RN(448 ss)
// (an overflow of |x| * 2^64 to infinity clamps too): below hi nothing
// changes, so the quotient is the IEEE one and at most hi / ss < 448 (1 + 2^-23);
// at or above hi the true quotient is at least 448 (1 - 2^-24), above E4M3FN's
// last rounding boundary 432, and so is that of hi itself. Either way the code
// is the saturating RNE code of the IEEE quotient, and every quotient handed
// to the conversion stays within the range where the hardware conversion is
// exact (|q| <= 464).
MXQ_HD float fp8_static_quotient(float x_abs, const Fp8Row& r) {
  float xs = fminf(x_abs * r.pre, r.hi);
  float q0 = xs * r.y;
  float rem = __builtin_fmaf(-q0, r.ss, xs);
  return __builtin_fmaf(rem, r.y, q0);
}

// E4M3FN code of a bf16 element under a static scale (s == 0: signed zero).
MXQ_HD uint32_t fp8_static_code_bf16(uint32_t bits16, const Fp8Row& r) {
  const uint32_t sign = (bits16 >> 8) & 0x80u;
  if (r.s == 0.0f) return sign;
  return e4m3fn_code(fp8_static_quotient(as_float((bits16 & 0x7FFFu) << 16), r)) | sign;
}

// --------------------------------------------------------------- bf16 -----

// fp32 -> bf16 bits, round half to even (finite inputs; NaN stays NaN).
MXQ_HD uint32_t bf16_rne(float f) {
  uint32_t b = as_uint(f);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return ((b >> 16) | 0x40u) & 0xFFFFu;
  return ((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16) & 0xFFFFu;
}

// tanh-GELU in fp32: 0.5 y (1 + tanh(sqrt(2/pi) (y + 0.044715 y^3))).
MXQ_HD float gelu_tanh(float y) {
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  float u = c * (y + 0.044715f * y * y * y);
  return 0.5f * y * (1.0f + tanhf(u));
}

}  // namespace mxq
