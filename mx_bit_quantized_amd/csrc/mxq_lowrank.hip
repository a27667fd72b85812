// mxq_lowrank.hip - SVDQuant's 16-bit low-rank branch beside the quantized
// product (section "Mixed-Precision selection" and its note, and the
// SVDQuant rows of "Results", of the page "Quark Mixed-Precision Quantization
// for Wan2.2 Video Generation on AMD Instinct GPUs"): for W ~ L2 L1^T + R,
//   T = RN_bf16(x L1)                       (lowrank_down_kernel)
//   y = RN_bf16(epilogue(y_pre + T L2^T))   (lowrank_up_kernel)
// with y_pre the quantized product Q(x) Q(R)^T (+ bias) in bf16. Both are
// bf16 contractions on the matrix cores (v_mfma_f32_32x32x16_bf16, fp32
// accumulation). The down projection reads x once (HBM-bound); the up one
// reads and writes y once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "mxq_convert.h"
#include "mxq_device.h"
#include "mxq_internal.h"

namespace mxq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// One 32 x 32 MFMA tile: D[i][j] = sum_k A[i][k] B[j][k] over k < 16. Lane l
// gives A row l % 32 and B row l % 32, k = 8 (l / 32) .. + 7 of each; its
// result registers q hold D[8 (q / 4) + 4 (l / 32) + q % 4][l % 32].
//
// Down projection: A = L1^T rows (rank index), B = x rows (tokens), so a lane
// ends with 16 rank values of one token. The contraction order is free, so
// MFMA k-slot (h, e) of super-step k0 and step s (0..3) is element
// k0 + 32 h + 8 s + e: each lane reads 64 contiguous bytes of its row per
// super-step, 16 at a time. A workgroup (4 waves) owns 32 tokens; its waves
// take contiguous quarters of K and fold their partial sums through LDS.
constexpr int kLrWaves = 4;

template <int R>  // rank / 32
__global__ __launch_bounds__(64 * kLrWaves) void lowrank_down_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                                     int64_t K, const uint16_t* __restrict__ l1t,
                                                                     uint16_t* __restrict__ t) {
  __shared__ float red[kLrWaves - 1][R][16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 31, h = lane >> 5;
  const int64_t row = (int64_t)blockIdx.x * 32 + r;
  const bool row_ok = row < M;
  const uint16_t* xr = x + (row_ok ? row : 0) * K + 32 * h;
  const int64_t steps = K / 64;
  const int64_t s_begin = steps * wave / kLrWaves, s_end = steps * (wave + 1) / kLrWaves;
  v16f_t acc[R];
#pragma unroll
  for (int q = 0; q < R; ++q) acc[q] = v16f_t{};
  for (int64_t st = s_begin; st < s_end; ++st) {
    const int64_t k0 = st * 64;
    uint4 xv[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
      xv[s] = row_ok ? reinterpret_cast<const uint4*>(xr + k0)[s] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int q = 0; q < R; ++q) {
        const uint4 lv = *reinterpret_cast<const uint4*>(l1t + (int64_t)(32 * q + r) * K + k0 + 32 * h + 8 * s);
        acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(lv), as_bf16x8(xv[s]), acc[q], 0, 0, 0);
      }
  }
  if (wave > 0) {
#pragma unroll
    for (int q = 0; q < R; ++q)
#pragma unroll
      for (int i = 0; i < 16; ++i) red[wave - 1][q][i][lane] = acc[q][i];
  }
  __syncthreads();
  if (wave != 0 || !row_ok) return;
  const int64_t rank = 32 * R;
#pragma unroll
  for (int q = 0; q < R; ++q) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int w = 0; w < kLrWaves - 1; ++w) acc[q][i] += red[w][q][i][lane];
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      const uint2 v = make_uint2(pack_bf16(acc[q][4 * t4], acc[q][4 * t4 + 1]),
                                 pack_bf16(acc[q][4 * t4 + 2], acc[q][4 * t4 + 3]));
      *reinterpret_cast<uint2*>(t + row * rank + 32 * q + 8 * t4 + 4 * h) = v;
    }
  }
}

// Up projection: A = L2 rows (output columns), B = T rows (tokens); a wave
// owns 32 tokens x 128 columns (four 32 x 32 tiles), r / 16 MFMA steps per
// tile. A lane ends with 16 columns of one token: 4 runs of 4 consecutive
// columns, which it reads from y_pre and writes to y (8 bytes each), so y may
// be y_pre itself. Rows past M are neither read nor written.
template <int S, bool GELU>  // S = rank / 16
__global__ __launch_bounds__(256) void lowrank_up_kernel(const uint16_t* __restrict__ y_pre,
                                                         const uint16_t* __restrict__ t,
                                                         const uint16_t* __restrict__ l2, int64_t M, int64_t N,
                                                         uint16_t* y) {
  const int lane = threadIdx.x & 63;
  const int64_t wave_id = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t strips = (N + 127) / 128;
  const int64_t row0 = wave_id / strips * 32, col0 = wave_id % strips * 128;
  if (row0 >= M) return;  // whole waves only: no barrier follows
  const int r = lane & 31, h = lane >> 5;
  const int64_t row = row0 + r;
  const bool row_ok = row < M;
  constexpr int64_t rank = 16 * S;
  uint4 tb[S];
#pragma unroll
  for (int s = 0; s < S; ++s)
    tb[s] = row_ok ? *reinterpret_cast<const uint4*>(t + row * rank + 16 * s + 8 * h) : make_uint4(0, 0, 0, 0);
  for (int c = 0; c < 4; ++c) {
    const int64_t n0 = col0 + 32 * c;
    if (n0 >= N) break;
    v16f_t acc = {};
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const uint4 a = *reinterpret_cast<const uint4*>(l2 + (n0 + r) * rank + 16 * s + 8 * h);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(tb[s]), acc, 0, 0, 0);
    }
    if (!row_ok) continue;
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      const int64_t n = n0 + 8 * t4 + 4 * h;
      const uint2 p = *reinterpret_cast<const uint2*>(y_pre + row * N + n);
      float v[4] = {as_float(p.x << 16) + acc[4 * t4], as_float(p.x & 0xFFFF0000u) + acc[4 * t4 + 1],
                    as_float(p.y << 16) + acc[4 * t4 + 2], as_float(p.y & 0xFFFF0000u) + acc[4 * t4 + 3]};
      if constexpr (GELU) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = gelu_tanh_dev(v[i]);
      }
      *reinterpret_cast<uint2*>(y + row * N + n) = make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
    }
  }
}

hipError_t launch_lowrank_down(const void* x, int64_t M, int64_t K, const void* l1t, int64_t r, void* t,
                               hipStream_t s) {
  const dim3 grid((unsigned)((M + 31) / 32)), block(64 * kLrWaves);
  const auto* xs = static_cast<const uint16_t*>(x);
  const auto* ls = static_cast<const uint16_t*>(l1t);
  auto* ts = static_cast<uint16_t*>(t);
  switch (r / 32) {
    case 1: hipLaunchKernelGGL(lowrank_down_kernel<1>, grid, block, 0, s, xs, M, K, ls, ts); break;
    case 2: hipLaunchKernelGGL(lowrank_down_kernel<2>, grid, block, 0, s, xs, M, K, ls, ts); break;
    case 3: hipLaunchKernelGGL(lowrank_down_kernel<3>, grid, block, 0, s, xs, M, K, ls, ts); break;
    default: hipLaunchKernelGGL(lowrank_down_kernel<4>, grid, block, 0, s, xs, M, K, ls, ts); break;
  }
  return hipGetLastError();
}

hipError_t launch_lowrank_up(const void* y_pre, const void* t, const void* l2, int64_t M, int64_t N, int64_t r,
                             int epilogue, void* y, hipStream_t s) {
  const int64_t waves = (M + 31) / 32 * ((N + 127) / 128);
  const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  const auto* yp = static_cast<const uint16_t*>(y_pre);
  const auto* ts = static_cast<const uint16_t*>(t);
  const auto* ls = static_cast<const uint16_t*>(l2);
  auto* ys = static_cast<uint16_t*>(y);
  auto go = [&](auto s_tag, auto g_tag) {
    hipLaunchKernelGGL((lowrank_up_kernel<decltype(s_tag)::value, decltype(g_tag)::value>), grid, block, 0, s,
                       yp, ts, ls, M, N, ys);
  };
  auto by_rank = [&](auto g_tag) {
    switch (r / 32) {
      case 1: go(std::integral_constant<int, 2>{}, g_tag); break;
      case 2: go(std::integral_constant<int, 4>{}, g_tag); break;
      case 3: go(std::integral_constant<int, 6>{}, g_tag); break;
      default: go(std::integral_constant<int, 8>{}, g_tag); break;
    }
  };
  if (epilogue == 1) by_rank(std::true_type{});
  else by_rank(std::false_type{});
  return hipGetLastError();
}

}  // namespace mxq
