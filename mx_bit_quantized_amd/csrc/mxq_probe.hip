// mxq_probe.hip - measurement kernels for the benchmark's roofline
// denominators (not part of the quantized linear): the rate the scaled MFMA
// instruction of the GEMMs reaches with nothing else running, on random
// operands, and a plain device copy.
//
// MFMA probe: every wave of a full-chip grid keeps 16 independent 32x32
// accumulator tiles and issues v_mfma_scale_f32_32x32x64_f8f6f4 on them in
// turn, like a GEMM's 4 x 4 tile of MFMAs: A fragment i for tiles 4i .. 4i+3,
// B fragment j for tiles j, 4 + j, ..., both rotating by one every round, from
// 4 random A and 4 random B fragments per lane (different for every lane and
// wave) with random E8M0 scales near 2^0, so consecutive instructions see
// different bits as in a GEMM. Operand format
// FP4 x FP4 (the W4A4 product) or FP8 x FP4 (W4A8). One wave per SIMD: the
// instruction issues every 32 (FP4) or 64 (FP8) cycles when the pipe is fed.
// Wave 0 of workgroup 0 also records s_memtime at its start and end, so the
// host gets the shader clock over the run.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

template <int FMT_B>  // 4: FP4 x FP4, 0: FP4 (A) x FP8 (B)
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void mfma_probe_kernel(
    const uint4* __restrict__ rnd, int iters, float* __restrict__ out, uint64_t* __restrict__ clk) {
  const int tid = blockIdx.x * 256 + threadIdx.x;
  const int nthreads = gridDim.x * 256;
  v8i A[4], B[4];
  uint32_t sa[4], sb[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 a = rnd[(2 * q) * nthreads + tid];
    const uint4 b = rnd[(2 * q + 1) * nthreads + tid];
    const uint4 c = rnd[(16 + q) * nthreads + tid];
    A[q] = v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    if constexpr (FMT_B == 4)
      B[q] = v8i{(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
    else
      B[q] = v8i{(int)b.x, (int)b.y, (int)b.z, (int)b.w, (int)c.x, (int)c.y, (int)c.z, (int)c.w};
    // E8M0 scale bytes in 2^-4 .. 2^3 (bytes 123 .. 130)
    sa[q] = 0x7B7B7B7Bu + (c.x & 0x07070707u);
    sb[q] = 0x7B7B7B7Bu + (c.y & 0x07070707u);
  }
  v16f acc[16];
#pragma unroll
  for (int s = 0; s < 16; ++s) acc[s] = v16f{};
  uint64_t t0 = 0;
  if (tid == 0) t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const int i = ((s >> 2) + r) & 3, j = ((s & 3) + r) & 3;
        acc[s] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[i], B[j], acc[s], 4, FMT_B, 0, (int)sa[i], 0,
                                                                 (int)sb[j]);
      }
  }
  float sum = 0.0f;
#pragma unroll
  for (int s = 0; s < 16; ++s)
#pragma unroll
    for (int e = 0; e < 16; ++e) sum += acc[s][e];
  out[tid] = sum;
  if (tid == 0) {
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    clk[0] = t1 - t0;
  }
}

// Each thread moves 4 words per round, all four loads issued before the
// stores; consecutive threads take consecutive words. n: a multiple of 1024.
__global__ __launch_bounds__(256) void copy_probe_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                         int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 1024;
  for (int64_t base = (int64_t)blockIdx.x * 1024 + threadIdx.x; base < n; base += stride) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = src[base + 256 * u];
#pragma unroll
    for (int u = 0; u < 4; ++u) dst[base + 256 * u] = v[u];
  }
}

}  // namespace mxq

extern "C" {

// Random operand words the MFMA probe needs: 24 uint4 per thread of its grid.
size_t mxq_probe_mfma_words(int grid) { return (size_t)24 * (size_t)grid * 256; }

// MFMA probe: `grid` workgroups of 256 threads, `iters` rounds of 128 MFMAs
// per wave. rnd: device uint4 [mxq_probe_mfma_words(grid)] of random bits;
// out: device float [grid * 256]; clk: device uint64 (shader clocks of wave 0).
// b_fp8 = 0: FP4 x FP4; 1: FP4 x FP8. Returns a hipError_t value.
int mxq_probe_mfma(int b_fp8, int grid, int iters, const void* rnd, float* out, uint64_t* clk, hipStream_t s) {
  if (b_fp8)
    hipLaunchKernelGGL(mxq::mfma_probe_kernel<0>, dim3(grid), dim3(256), 0, s, static_cast<const uint4*>(rnd), iters,
                       out, clk);
  else
    hipLaunchKernelGGL(mxq::mfma_probe_kernel<4>, dim3(grid), dim3(256), 0, s, static_cast<const uint4*>(rnd), iters,
                       out, clk);
  return (int)hipGetLastError();
}

// Device copy of n uint4 words, n a multiple of 1024 (src and dst device,
// 16-byte aligned).
int mxq_probe_copy(const void* src, void* dst, int64_t n, int grid, hipStream_t s) {
  hipLaunchKernelGGL(mxq::copy_probe_kernel, dim3(grid), dim3(256), 0, s, static_cast<const uint4*>(src),
                     static_cast<uint4*>(dst), n);
  return (int)hipGetLastError();
}

}  // extern "C"
