// mxq_device.h - device-only helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace mxq {

// tanh-GELU in fp32, 0.5 y (1 + tanh(u)) with u = sqrt(2/pi) (y + 0.044715 y^3),
// written as y / (1 + exp(-2u)) and exp(-2u) = 2^(y (c0 + c1 y^2)) with the
// constants folded: 5 VALU operations and 2 transcendental ones per element.
__device__ __forceinline__ float gelu_tanh_dev(float y) {
  constexpr float kL = -2.0f * 1.4426950408889634f * 0.7978845608028654f;  // -2 log2(e) sqrt(2/pi)
  const float e = __builtin_amdgcn_exp2f(y * __builtin_fmaf(y * y, kL * 0.044715f, kL));
  return y * __builtin_amdgcn_rcpf(1.0f + e);
}

}  // namespace mxq
