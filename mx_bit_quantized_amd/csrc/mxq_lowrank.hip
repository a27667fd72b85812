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

// ---- down projection: T = RN_bf16(x L1) ---------------------------------
//
// A workgroup (4 waves) owns 64 rows of x and walks K in chunks of 128. Each
// chunk of x (64 x 128 bf16, 16 KiB) and of L1^T (r x 128) is loaded with
// row-contiguous 16-byte loads (whole 256-byte row runs per instruction) into
// registers two chunks ahead, then through LDS to the matrix cores. Wave w takes k = 32 w .. 32 w + 31 of the chunk (two MFMA
// steps) for every output tile (2 row tiles x r/32 rank tiles), with A = L1^T
// rows and B = x rows, so a lane ends with 16 rank values of one row; the
// four waves' partial sums are added through LDS at the end.
constexpr int kDnRows = 64;
constexpr int kDnKc = 128;
constexpr int kDnPitch = kDnKc * 2 + 16;  // bytes per LDS row: 16-byte reads of 16 rows hit 16 bank groups

//
// QUANT: the same pass also writes the W4A4 activation of x (the MXFP4
// quantizer's codes and scales, byte for byte): once a chunk is in LDS and its
// MFMAs are issued, thread u quantizes block u % 4 of chunk row u / 4 (32
// elements: block amax, scale byte, 16 code bytes by the scaled conversion).
// The chunk is one code panel: each wave stores 16 rows x 64 bytes of codes,
// 1 KiB of consecutive memory, and the rows' scale dwords.
template <int R, bool QUANT>  // rank / 32; with the activation quantizer
__global__ __launch_bounds__(256) void lowrank_down_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                          const uint16_t* __restrict__ l1t,
                                                          uint16_t* __restrict__ t, uint8_t* __restrict__ codes,
                                                          uint32_t* __restrict__ scales) {
  constexpr int RANK = 32 * R;
  constexpr int XB = kDnRows * kDnPitch, LB = RANK * kDnPitch;
  constexpr int RED = 3 * 16 * 64 * 4;  // one output tile's partial sums of waves 1..3
  __shared__ __attribute__((aligned(16))) uint8_t lds[(XB + LB) > RED ? (XB + LB) : RED];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, h = lane >> 5;
  const int64_t row0 = (int64_t)blockIdx.x * kDnRows;
  // loader mapping: 16-byte chunk lc = tid % 16 of row lr = tid / 16 (+ 16 i)
  const int lc = tid & 15, lr = tid >> 4;
  constexpr int XN = kDnRows / 16, LN = RANK / 16;  // 16-byte loads per thread and chunk
  // two chunks in flight: register sets A and B alternate
  uint4 xa[XN], la[LN], xb[XN], lb[LN];
  auto load = [&](uint4 (&xr)[XN], uint4 (&lrg)[LN], int64_t k0) {
#pragma unroll
    for (int i = 0; i < XN; ++i) {
      const int rr = lr + 16 * i;
      const int64_t row = row0 + rr;
      xr[i] = (rr < kDnRows && row < M) ? *reinterpret_cast<const uint4*>(x + row * K + k0 + 8 * lc)
                                        : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < LN; ++i) {
      const int rr = lr + 16 * i;
      lrg[i] = rr < RANK ? *reinterpret_cast<const uint4*>(l1t + (int64_t)rr * K + k0 + 8 * lc) : make_uint4(0, 0, 0, 0);
    }
  };
  v16f_t acc[2][R];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int q = 0; q < R; ++q) acc[a][q] = v16f_t{};
  // chunk k0 from (xr, lrg): into LDS, refill the registers with chunk k0 + 2 Kc, multiply
  auto body = [&](uint4 (&xr)[XN], uint4 (&lrg)[LN], int64_t k0) {
    __syncthreads();  // the previous chunk's reads are done
#pragma unroll
    for (int i = 0; i < XN; ++i)
      if (lr + 16 * i < kDnRows) *reinterpret_cast<uint4*>(lds + (lr + 16 * i) * kDnPitch + 16 * lc) = xr[i];
#pragma unroll
    for (int i = 0; i < LN; ++i)
      if (lr + 16 * i < RANK) *reinterpret_cast<uint4*>(lds + XB + (lr + 16 * i) * kDnPitch + 16 * lc) = lrg[i];
    __syncthreads();
    if (k0 + 2 * kDnKc < K) load(xr, lrg, k0 + 2 * kDnKc);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int kb = (32 * wave + 16 * s + 8 * h) * 2;  // byte offset of the lane's 8 elements
      uint4 bx[2], al[R];
#pragma unroll
      for (int a = 0; a < 2; ++a) bx[a] = *reinterpret_cast<const uint4*>(lds + (32 * a + r) * kDnPitch + kb);
#pragma unroll
      for (int q = 0; q < R; ++q) al[q] = *reinterpret_cast<const uint4*>(lds + XB + (32 * q + r) * kDnPitch + kb);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int q = 0; q < R; ++q)
          acc[a][q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(al[q]), as_bf16x8(bx[a]), acc[a][q], 0, 0, 0);
    }
    if constexpr (QUANT) {
      const int qr = tid >> 2, qb = tid & 3;
      const uint8_t* src = lds + qr * kDnPitch + qb * 64;
      uint4 c[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) c[i] = *reinterpret_cast<const uint4*>(src + 16 * i);
      const uint32_t am = umax(umax(chunk_amax(c[0]), chunk_amax(c[1])), umax(chunk_amax(c[2]), chunk_amax(c[3])));
      const uint32_t sb = mx_scale_byte(am);
      const uint4 cw = make_uint4(pack8_fp4(c[0], sb), pack8_fp4(c[1], sb), pack8_fp4(c[2], sb), pack8_fp4(c[3], sb));
      // the row's four scale bytes, from the quad's lanes (row = lane / 4)
      const uint32_t s1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)sb, 0x39, 0xF, 0xF, false);  // lane + 1
      const uint32_t s2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)sb, 0x4E, 0xF, 0xF, false);  // lane + 2
      const uint32_t s3 = (uint32_t)__builtin_amdgcn_mov_dpp((int)sb, 0x93, 0xF, 0xF, false);  // lane + 3
      const int64_t row = row0 + qr, p = k0 >> 7;
      if (row < M) {
        *reinterpret_cast<uint4*>(codes + p * 64 * M + row * 64 + qb * 16) = cw;
        if (qb == 0) scales[p * M + row] = sb | (s1 << 8) | (s2 << 16) | (s3 << 24);
      }
    }
  };
  load(xa, la, 0);
  if (kDnKc < K) load(xb, lb, kDnKc);
  for (int64_t k0 = 0; k0 < K; k0 += 2 * kDnKc) {
    body(xa, la, k0);
    if (k0 + kDnKc < K) body(xb, lb, k0 + kDnKc);
  }
  // fold the waves' partial sums tile by tile through LDS (every wave takes
  // part in every barrier; wave 0 adds and stores)
  float* red = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int64_t row = row0 + 32 * a + r;
#pragma unroll
    for (int q = 0; q < R; ++q) {
      __syncthreads();
      if (wave > 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) red[((wave - 1) * 16 + i) * 64 + lane] = acc[a][q][i];
      }
      __syncthreads();
      if (wave != 0) continue;
#pragma unroll
      for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int w = 0; w < 3; ++w) acc[a][q][i] += red[(w * 16 + i) * 64 + lane];
      if (row < M) {
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4)
          *reinterpret_cast<uint2*>(t + row * RANK + 32 * q + 8 * t4 + 4 * h) =
              make_uint2(pack_bf16(acc[a][q][4 * t4], acc[a][q][4 * t4 + 1]),
                         pack_bf16(acc[a][q][4 * t4 + 2], acc[a][q][4 * t4 + 3]));
      }
    }
  }
}

// ---- up projection: y = RN_bf16(epilogue(y_pre + T L2^T)) ----------------
//
// A wave owns 32 rows x 128 columns, in two passes of 64 columns: two MFMA
// tiles with A = L2 rows (columns of y) and B = T rows, r / 16 steps each.
// The sums go through a per-wave LDS area as a row-major 32 x 64 fp32 block;
// the lanes then read 8 consecutive columns each, 8 rows x 64 columns per
// instruction, add y_pre, apply the epilogue and store 16 bytes: whole
// 128-byte row runs per instruction. The wave's y_pre loads (16 bytes each,
// same lane-to-element map) are all issued before the MFMAs. Every element is
// read and written by one lane, so y may be y_pre. Rows past M are neither
// read nor written.
constexpr int kUpPitch = 64 * 4 + 16;  // bytes per LDS row of the 32 x 64 fp32 block

template <int S, bool GELU>  // S = rank / 16
__global__ __launch_bounds__(256) void lowrank_up_kernel(const uint16_t* __restrict__ y_pre,
                                                         const uint16_t* __restrict__ t,
                                                         const uint16_t* __restrict__ l2, int64_t M, int64_t N,
                                                         uint16_t* y) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[4][32 * kUpPitch];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t wave_id = (int64_t)blockIdx.x * 4 + wave;
  const int64_t strips = (N + 127) / 128;
  const int64_t row0 = wave_id / strips * 32, col0 = wave_id % strips * 128;
  if (row0 >= M) return;  // whole waves only; the LDS area is the wave's own, no barrier follows
  const int r = lane & 31, h = lane >> 5;
  constexpr int64_t rank = 16 * S;
  uint8_t* blk = lds[wave];
  const int64_t trow = row0 + r;
  const int lc = lane & 7;  // 8-column chunk of the pass
  // both passes' y_pre loads go out first, so that they are in flight during the MFMAs
  uint4 pre[2][4];
#pragma unroll
  for (int pass = 0; pass < 2; ++pass)
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int64_t row = row0 + 8 * it + (lane >> 3), n = col0 + 64 * pass + 8 * lc;
      pre[pass][it] =
          (row < M && n < N) ? *reinterpret_cast<const uint4*>(y_pre + row * N + n) : make_uint4(0, 0, 0, 0);
    }
  uint4 tb[S];
#pragma unroll
  for (int s = 0; s < S; ++s)
    tb[s] = trow < M ? *reinterpret_cast<const uint4*>(t + trow * rank + 16 * s + 8 * h) : make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    for (int c = 0; c < 2; ++c) {
      const int64_t n0 = col0 + 64 * pass + 32 * c;
      v16f_t acc = {};
      if (n0 < N) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
          const uint4 a = *reinterpret_cast<const uint4*>(l2 + (n0 + r) * rank + 16 * s + 8 * h);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(tb[s]), acc, 0, 0, 0);
        }
      }
      // D[n][m] -> block[m = r][n = 32 c + 8 (q / 4) + 4 h + q % 4]
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4)
        *reinterpret_cast<float4*>(blk + r * kUpPitch + (32 * c + 8 * t4 + 4 * h) * 4) =
            make_float4(acc[4 * t4], acc[4 * t4 + 1], acc[4 * t4 + 2], acc[4 * t4 + 3]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int rr = 8 * it + (lane >> 3);
      const int64_t row = row0 + rr, n = col0 + 64 * pass + 8 * lc;
      if (row >= M || n >= N) continue;
      const float4 lo = *reinterpret_cast<const float4*>(blk + rr * kUpPitch + lc * 32);
      const float4 hi = *reinterpret_cast<const float4*>(blk + rr * kUpPitch + lc * 32 + 16);
      const uint4 p = pre[pass][it];
      float v[8] = {as_float(p.x << 16) + lo.x, as_float(p.x & 0xFFFF0000u) + lo.y,
                    as_float(p.y << 16) + lo.z, as_float(p.y & 0xFFFF0000u) + lo.w,
                    as_float(p.z << 16) + hi.x, as_float(p.z & 0xFFFF0000u) + hi.y,
                    as_float(p.w << 16) + hi.z, as_float(p.w & 0xFFFF0000u) + hi.w};
      if constexpr (GELU) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = gelu_tanh_dev(v[i]);
      }
      *reinterpret_cast<uint4*>(y + row * N + n) =
          make_uint4(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7]));
    }
    // the next pass overwrites the block: its writes stay behind these reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

hipError_t launch_lowrank_down(const void* x, int64_t M, int64_t K, const void* l1t, int64_t r, void* t,
                               void* codes, void* scales, hipStream_t s) {
  const dim3 grid((unsigned)((M + kDnRows - 1) / kDnRows)), block(256);
  const auto* xs = static_cast<const uint16_t*>(x);
  const auto* ls = static_cast<const uint16_t*>(l1t);
  auto* ts = static_cast<uint16_t*>(t);
  auto* cs = static_cast<uint8_t*>(codes);
  auto* ss = static_cast<uint32_t*>(scales);
  auto go = [&](auto r_tag, auto q_tag) {
    hipLaunchKernelGGL((lowrank_down_kernel<decltype(r_tag)::value, decltype(q_tag)::value>), grid, block, 0, s, xs,
                       M, K, ls, ts, cs, ss);
  };
  auto by_rank = [&](auto q_tag) {
    switch (r / 32) {
      case 1: go(std::integral_constant<int, 1>{}, q_tag); break;
      case 2: go(std::integral_constant<int, 2>{}, q_tag); break;
      case 3: go(std::integral_constant<int, 3>{}, q_tag); break;
      default: go(std::integral_constant<int, 4>{}, q_tag); break;
    }
  };
  if (codes != nullptr) by_rank(std::true_type{});
  else by_rank(std::false_type{});
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
