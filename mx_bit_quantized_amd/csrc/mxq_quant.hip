// mxq_quant.hip - bf16 -> MXFP4 and bf16 -> FP8 per-token quantizers (gfx950).
//
// MXFP4 (weights offline, W4A4 activations on the fly) and FP8 E4M3FN
// per-token (W4A8 activations), section "Quantization formats" of the page
// "Quark Mixed-Precision Quantization for Wan2.2 Video Generation on AMD
// Instinct GPUs". Both kernels are HBM-bound streams: one read of the bf16
// rows, one write of the codes and scales.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq_convert.h"
#include "mxq_internal.h"

namespace mxq {

// ------------------------------------------------------------ MXFP4 -------
//
// Mapping: a wave walks one row at a time; each lane owns one 16-byte chunk
// (8 bf16) per step, so four neighbouring lanes hold one 32-element block and
// sixteen lanes one 128-element group. A step reads 1 KiB contiguous per wave
// and writes 256 contiguous bytes of codes (4 per lane). The block amax is a
// max over the magnitude bit patterns (sign cleared) across the 4 lanes -
// exact for finite bf16, no float compare, no denormal flush.
//
// Scales are stored group-major, [ceil(K/128)][rows][4]: the four E8M0 bytes
// of the blocks of one 128-element group of one row form one dword, and the
// dwords of all rows for one group are contiguous. The GEMM then fetches the
// scales of a 256-row tile for one K stage as 1 KiB of consecutive memory.
// The first lane of each group assembles the dword from the four block
// leaders and writes it; bytes of blocks past K/32 in a ragged last group are
// written as zero.

__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  v = umax(v, (uint32_t)__shfl_xor((int)v, 1));
  v = umax(v, (uint32_t)__shfl_xor((int)v, 2));
  return v;
}

__device__ __forceinline__ uint32_t pack8_fp4(const uint4 c, float inv) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  uint32_t out = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t lo = e2m1_code_bf16(w[i] & 0xFFFFu, inv);
    uint32_t hi = e2m1_code_bf16(w[i] >> 16, inv);
    out |= (lo | (hi << 4)) << (8 * i);
  }
  return out;
}

__device__ __forceinline__ uint32_t chunk_amax(const uint4 c) {
  uint32_t m0 = umax(c.x & 0x7FFFu, (c.x >> 16) & 0x7FFFu);
  uint32_t m1 = umax(c.y & 0x7FFFu, (c.y >> 16) & 0x7FFFu);
  uint32_t m2 = umax(c.z & 0x7FFFu, (c.z >> 16) & 0x7FFFu);
  uint32_t m3 = umax(c.w & 0x7FFFu, (c.w >> 16) & 0x7FFFu);
  return umax(umax(m0, m1), umax(m2, m3));
}

constexpr int kQuantWaves = 4;  // waves per workgroup

__global__ __launch_bounds__(64 * kQuantWaves) void mxfp4_quant_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t K, int64_t ld,
    uint8_t* __restrict__ codes, uint32_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t wave_id = (int64_t)blockIdx.x * kQuantWaves + (threadIdx.x >> 6);
  const int64_t n_waves = (int64_t)gridDim.x * kQuantWaves;
  const int64_t chunks = K >> 3;  // 8 bf16 per chunk, 4 chunks per block
  for (int64_t row = wave_id; row < rows; row += n_waves) {
    const uint4* src = reinterpret_cast<const uint4*>(x + row * ld);
    uint32_t* dst = reinterpret_cast<uint32_t*>(codes + row * (K >> 1));
    for (int64_t c0 = 0; c0 < chunks; c0 += 64) {
      const int64_t c = c0 + lane;
      // chunks is a multiple of 4 and c0 of 64, so a whole 4-lane block is
      // either in range or out of range: the shuffles stay uniform per block.
      const bool ok = c < chunks;
      uint4 v = ok ? src[c] : make_uint4(0, 0, 0, 0);
      uint32_t amax = quad_max(chunk_amax(v));
      uint32_t sb = mx_scale_byte(amax);
      uint32_t packed = pack8_fp4(v, mx_inv_scale(sb));
      // gather the 4 block scales of this lane's 128-element group into its
      // first lane (block leaders sit at lanes +0, +4, +8, +12); out-of-range
      // blocks contribute zero bytes
      const uint32_t mine = ok ? sb : 0u;
      const uint32_t s1 = (uint32_t)__shfl_down((int)mine, 4);
      const uint32_t s2 = (uint32_t)__shfl_down((int)mine, 8);
      const uint32_t s3 = (uint32_t)__shfl_down((int)mine, 12);
      if (ok) {
        dst[c] = packed;
        if ((lane & 15) == 0) scales[(c >> 4) * rows + row] = mine | (s1 << 8) | (s2 << 16) | (s3 << 24);
      }
    }
  }
}

// ------------------------------------------------------------- FP8 --------
//
// One wave per row: pass 1 reduces the row amax (magnitude bit patterns) over
// the wave, then every lane derives the same scale; pass 2 re-reads the row
// (an L2 hit for rows of tens of KiB) and writes 8 E4M3FN codes per chunk.

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = umax(v, (uint32_t)__shfl_xor((int)v, off));
  return v;
}

__device__ __forceinline__ uint2 pack8_fp8(const uint4 c, const Fp8Row& r) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  uint32_t out[2] = {0, 0};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t lo = fp8_code_bf16(w[i] & 0xFFFFu, r);
    uint32_t hi = fp8_code_bf16(w[i] >> 16, r);
    out[i >> 1] |= (lo | (hi << 8)) << (16 * (i & 1));
  }
  return make_uint2(out[0], out[1]);
}

__global__ __launch_bounds__(64 * kQuantWaves) void fp8_quant_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t K, int64_t ld,
    uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t wave_id = (int64_t)blockIdx.x * kQuantWaves + (threadIdx.x >> 6);
  const int64_t n_waves = (int64_t)gridDim.x * kQuantWaves;
  const int64_t chunks = K >> 3;
  for (int64_t row = wave_id; row < rows; row += n_waves) {
    const uint4* src = reinterpret_cast<const uint4*>(x + row * ld);
    uint32_t amax = 0;
    for (int64_t c = lane; c < chunks; c += 64) amax = umax(amax, chunk_amax(src[c]));
    amax = wave_max(amax);
    const Fp8Row r = fp8_row_setup(amax);
    uint2* dst = reinterpret_cast<uint2*>(codes + row * K);
    for (int64_t c = lane; c < chunks; c += 64) dst[c] = pack8_fp8(src[c], r);
    if (lane == 0) scales[row] = r.s;
  }
}

// ------------------------------------------------------------ launch ------

static int grid_for_rows(int64_t rows) {
  int64_t blocks = (rows + kQuantWaves - 1) / kQuantWaves;
  const int64_t cap = 256 * 64;  // enough to fill 256 CUs many times; rows loop beyond
  return (int)(blocks < cap ? blocks : cap);
}

hipError_t launch_mxfp4_quant(const void* x, int64_t rows, int64_t K, int64_t ld,
                              void* codes, void* scales, hipStream_t s) {
  hipLaunchKernelGGL(mxfp4_quant_kernel, dim3(grid_for_rows(rows)), dim3(64 * kQuantWaves), 0, s,
                     static_cast<const uint16_t*>(x), rows, K, ld,
                     static_cast<uint8_t*>(codes), static_cast<uint32_t*>(scales));
  return hipGetLastError();
}

hipError_t launch_fp8_quant(const void* x, int64_t rows, int64_t K, int64_t ld,
                            void* codes, void* scales, hipStream_t s) {
  hipLaunchKernelGGL(fp8_quant_kernel, dim3(grid_for_rows(rows)), dim3(64 * kQuantWaves), 0, s,
                     static_cast<const uint16_t*>(x), rows, K, ld,
                     static_cast<uint8_t*>(codes), static_cast<float*>(scales));
  return hipGetLastError();
}

}  // namespace mxq
