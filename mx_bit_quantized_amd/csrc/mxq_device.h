// mxq_device.h - device-only helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq_convert.h"

namespace mxq {

// tanh-GELU in fp32, 0.5 y (1 + tanh(u)) with u = sqrt(2/pi) (y + 0.044715 y^3),
// written as y / (1 + exp(-2u)) and exp(-2u) = 2^(y (c0 + c1 y^2)) with the
// constants folded: 5 VALU operations and 2 transcendental ones per element.
__device__ __forceinline__ float gelu_tanh_dev(float y) {
  constexpr float kL = -2.0f * 1.4426950408889634f * 0.7978845608028654f;  // -2 log2(e) sqrt(2/pi)
  const float e = __builtin_amdgcn_exp2f(y * __builtin_fmaf(y * y, kL * 0.044715f, kL));
  return y * __builtin_amdgcn_rcpf(1.0f + e);
}

// MXFP4 block helpers (the quantizers' rule, OCP MX: scale byte from the
// block's largest magnitude, elements rounded by the scaled conversion).
//
// Largest magnitude bit pattern (sign cleared) of 8 bf16: exact for finite
// bf16, no float compare and no denormal flush.
__device__ __forceinline__ uint32_t chunk_amax(const uint4 c) {
  uint32_t m0 = umax(c.x & 0x7FFFu, (c.x >> 16) & 0x7FFFu);
  uint32_t m1 = umax(c.y & 0x7FFFu, (c.y >> 16) & 0x7FFFu);
  uint32_t m2 = umax(c.z & 0x7FFFu, (c.z >> 16) & 0x7FFFu);
  uint32_t m3 = umax(c.w & 0x7FFFu, (c.w >> 16) & 0x7FFFu);
  return umax(umax(m0, m1), umax(m2, m3));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// 8 bf16 -> 8 E2M1 codes (element 2t in the low nibble of byte t) of a block
// with scale byte sb, with gfx950's scaled conversion: it divides by the
// power of two whose exponent field is sb and rounds to nearest even,
// saturating at 6, keeping the sign (also of zeros). For every finite bf16
// and every scale byte of a block that can hold it this equals
// e2m1_code_bf16 (an exhaustive GPU test checks it).
__device__ __forceinline__ uint32_t pack8_fp4(const uint4 c, uint32_t sb) {
  const float scale = as_float(sb << 23);
  uint32_t out = 0;
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, __builtin_bit_cast(bf16x2_t, c.x), scale, 0);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, __builtin_bit_cast(bf16x2_t, c.y), scale, 1);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, __builtin_bit_cast(bf16x2_t, c.z), scale, 2);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, __builtin_bit_cast(bf16x2_t, c.w), scale, 3);
  return out;
}

}  // namespace mxq
