// mxq_select.hip - kernels of the calibration-driven block selection
// (section "Calibration-driven block selection" of the page "Quark
// Mixed-Precision Quantization for Wan2.2 Video Generation on AMD Instinct
// GPUs"): the signal and noise energies of a replayed layer output against
// the captured BF16 output, and a zero fill for the replay's running maxima.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq_convert.h"
#include "mxq_internal.h"

namespace mxq {

constexpr int kSqnrThreads = 256;

__device__ __forceinline__ void sqnr_add(uint32_t yb, uint32_t rb, double& sig, double& noise) {
  const double r = (double)as_float(rb << 16);
  const double d = (double)as_float(yb << 16) - r;
  sig = __builtin_fma(r, r, sig);
  noise = __builtin_fma(d, d, noise);
}

// sums[0] += sum r^2, sums[1] += sum (y - r)^2 over n bf16 pairs, in fp64
// (bf16 values and their squares are exact in fp64; the differences nearly
// always are). Each thread takes 8 elements per 16-byte load; the workgroup
// folds its sums through LDS and adds them with two fp64 atomics.
__global__ __launch_bounds__(kSqnrThreads) void sqnr_sum_kernel(const uint16_t* __restrict__ y,
                                                                const uint16_t* __restrict__ y_ref, int64_t n,
                                                                double* __restrict__ sums) {
  __shared__ double red[2][kSqnrThreads / 64];
  double sig = 0.0, noise = 0.0;
  const int64_t n8 = n >> 3;
  const int64_t stride = (int64_t)gridDim.x * kSqnrThreads;
  const int64_t t0 = (int64_t)blockIdx.x * kSqnrThreads + threadIdx.x;
  for (int64_t i = t0; i < n8; i += stride) {
    const uint4 a = reinterpret_cast<const uint4*>(y)[i];
    const uint4 b = reinterpret_cast<const uint4*>(y_ref)[i];
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sqnr_add(aw[j] & 0xFFFFu, bw[j] & 0xFFFFu, sig, noise);
      sqnr_add(aw[j] >> 16, bw[j] >> 16, sig, noise);
    }
  }
  for (int64_t i = (n8 << 3) + t0; i < n; i += stride) sqnr_add(y[i], y_ref[i], sig, noise);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    sig += __shfl_xor(sig, off);
    noise += __shfl_xor(noise, off);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    red[0][wave] = sig;
    red[1][wave] = noise;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double s = 0.0, e = 0.0;
#pragma unroll
    for (int w = 0; w < kSqnrThreads / 64; ++w) {
      s += red[0][w];
      e += red[1][w];
    }
    atomicAdd(&sums[0], s);
    atomicAdd(&sums[1], e);
  }
}

__global__ void fill_zero_kernel(uint32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

hipError_t launch_sqnr_sums(const void* y, const void* y_ref, int64_t n, double* sums, hipStream_t s) {
  int64_t blocks = (n / 8 + kSqnrThreads - 1) / kSqnrThreads;
  blocks = blocks < 2048 ? (blocks > 0 ? blocks : 1) : 2048;
  hipLaunchKernelGGL(sqnr_sum_kernel, dim3((unsigned)blocks), dim3(kSqnrThreads), 0, s,
                     static_cast<const uint16_t*>(y), static_cast<const uint16_t*>(y_ref), n, sums);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, int64_t n_words, hipStream_t s) {
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n_words + 255) / 256)), dim3(256), 0, s,
                     static_cast<uint32_t*>(p), n_words);
  return hipGetLastError();
}

}  // namespace mxq
