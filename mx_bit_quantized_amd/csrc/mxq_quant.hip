// mxq_quant.hip - bf16 -> MXFP4 and bf16 -> FP8 per-token quantizers (gfx950).
//
// MXFP4 (weights offline, W4A4 activations on the fly) and FP8 E4M3FN
// per-token (W4A8 activations), section "Quantization formats" of the page
// "Quark Mixed-Precision Quantization for Wan2.2 Video Generation on AMD
// Instinct GPUs". Both kernels are HBM-bound streams: one read of the bf16
// rows, one write of the codes and scales (rows longer than 14336 elements
// take a second read in the FP8 quantizer).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq_convert.h"
#include "mxq_internal.h"

namespace mxq {

// ------------------------------------------------------------ codes -------
//
// Codes are stored K-panel-major: K is cut into panels of 128 elements (the
// last one narrower when K % 128 != 0), and panel p holds every row's codes
// of elements 128p .. 128p + w_p - 1 contiguously, row after row. One GEMM
// stage of a 256-row tile is then one contiguous block. Byte offset of
// element k (a multiple of 8 here) of `row`, for codes of `bits` bits:
//   p * 128 * rows * bits / 8 + row * w_p * bits / 8 + (k - 128 p) * bits / 8.
__device__ __forceinline__ int64_t panel_offset(int64_t k, int64_t row, int64_t rows, int64_t K, int bits) {
  const int64_t p = k >> 7;
  const int64_t w = K - 128 * p < 128 ? K - 128 * p : 128;
  return ((p * 128 * rows + row * w + (k & 127)) * bits) >> 3;
}

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

__device__ __forceinline__ uint32_t chunk_amax(const uint4 c) {
  uint32_t m0 = umax(c.x & 0x7FFFu, (c.x >> 16) & 0x7FFFu);
  uint32_t m1 = umax(c.y & 0x7FFFu, (c.y >> 16) & 0x7FFFu);
  uint32_t m2 = umax(c.z & 0x7FFFu, (c.z >> 16) & 0x7FFFu);
  uint32_t m3 = umax(c.w & 0x7FFFu, (c.w >> 16) & 0x7FFFu);
  return umax(umax(m0, m1), umax(m2, m3));
}

constexpr int kQuantWaves = 4;  // waves per workgroup

// A wave converts a row in batches of B chunks per lane (B KiB per wave): all
// loads of a batch are issued before the first conversion, so each wave keeps
// that much of the stream in flight. The launcher picks B so that a row
// splits into equal batches of at most 16 chunks per lane.
template <int B>
__global__ __launch_bounds__(64 * kQuantWaves) void mxfp4_quant_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t K, int64_t ld,
    uint8_t* __restrict__ codes, uint32_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t wave_id = (int64_t)blockIdx.x * kQuantWaves + (threadIdx.x >> 6);
  const int64_t n_waves = (int64_t)gridDim.x * kQuantWaves;
  const int64_t chunks = K >> 3;  // 8 bf16 per chunk, 4 chunks per block
  for (int64_t row = wave_id; row < rows; row += n_waves) {
    const uint4* src = reinterpret_cast<const uint4*>(x + row * ld);
    for (int64_t c0 = 0; c0 < chunks; c0 += 64 * B) {
      uint4 v[B];
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const int64_t c = c0 + 64 * b + lane;
        v[b] = c < chunks ? src[c] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const int64_t c = c0 + 64 * b + lane;
        // chunks is a multiple of 4 and c - lane of 64, so a whole 4-lane
        // block is either in range or out of range: the shuffles stay
        // uniform per block.
        const bool ok = c < chunks;
        const uint32_t amax = quad_max(chunk_amax(v[b]));
        const uint32_t sb = mx_scale_byte(amax);
        const uint32_t packed = pack8_fp4(v[b], sb);
        // gather the 4 block scales of this lane's 128-element group into its
        // first lane (block leaders sit at lanes +0, +4, +8, +12);
        // out-of-range blocks contribute zero bytes
        const uint32_t mine = ok ? sb : 0u;
        const uint32_t s1 = (uint32_t)__shfl_down((int)mine, 4);
        const uint32_t s2 = (uint32_t)__shfl_down((int)mine, 8);
        const uint32_t s3 = (uint32_t)__shfl_down((int)mine, 12);
        if (ok) {
          *reinterpret_cast<uint32_t*>(codes + panel_offset(c * 8, row, rows, K, 4)) = packed;
          if ((lane & 15) == 0) scales[(c >> 4) * rows + row] = mine | (s1 << 8) | (s2 << 16) | (s3 << 24);
        }
      }
    }
  }
}

// ------------------------------------------------------------- FP8 --------
//
// One wave per row. Rows of up to 64 * 8 * MAXC elements are read once: the
// wave holds the whole row in registers (MAXC chunks per lane), reduces the
// row amax (magnitude bit patterns) over the wave, derives the scale and
// writes 8 E4M3FN codes per chunk. Longer rows take two passes: the amax,
// then a second read of the row to quantize it.

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = umax(v, (uint32_t)__shfl_xor((int)v, off));
  return v;
}

// Signed IEEE quotient x / s of a bf16 element: formed from |x| (rounding to
// nearest is symmetric; the FMA correction would lose the sign of -0) with
// x's sign attached. A row of zeros has s = 0: its quotients are signed zeros
// (the reciprocal is infinite there, and 0 * inf would be NaN).
__device__ __forceinline__ float fp8_signed_quotient(uint32_t bits16, const Fp8Row& r) {
  const float q = r.s == 0.0f ? 0.0f : fp8_quotient(as_float((bits16 & 0x7FFFu) << 16), r);
  return as_float(as_uint(q) | ((bits16 & 0x8000u) << 16));
}

// 8 bf16 -> 8 E4M3FN codes. The quotients are correctly rounded fp32 with
// |q| <= 448 (1 + 2^-22); gfx950's packed conversion rounds them to nearest
// even, signs and subnormals included: for every fp32 with |q| <= 464 it
// equals e4m3fn_code (an exhaustive GPU test checks it).
__device__ __forceinline__ uint2 pack8_fp8(const uint4 c, const Fp8Row& r) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  uint32_t out[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float q0 = fp8_signed_quotient(w[2 * i] & 0xFFFFu, r), q1 = fp8_signed_quotient(w[2 * i] >> 16, r);
    const float q2 = fp8_signed_quotient(w[2 * i + 1] & 0xFFFFu, r), q3 = fp8_signed_quotient(w[2 * i + 1] >> 16, r);
    uint32_t o = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
    o = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, (int)o, true);
    out[i] = o;
  }
  return make_uint2(out[0], out[1]);
}

template <int MAXC>
__global__ __launch_bounds__(64 * kQuantWaves) void fp8_quant_row_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t K, int64_t ld,
    uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t wave_id = (int64_t)blockIdx.x * kQuantWaves + (threadIdx.x >> 6);
  const int64_t n_waves = (int64_t)gridDim.x * kQuantWaves;
  const int chunks = (int)(K >> 3);
  for (int64_t row = wave_id; row < rows; row += n_waves) {
    const uint4* src = reinterpret_cast<const uint4*>(x + row * ld);
    uint4 v[MAXC];
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int c = 64 * i + lane;
      v[i] = c < chunks ? src[c] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < MAXC; ++i) amax = umax(amax, chunk_amax(v[i]));
    amax = wave_max(amax);
    const Fp8Row r = fp8_row_setup(amax);
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int c = 64 * i + lane;
      if (c < chunks) *reinterpret_cast<uint2*>(codes + panel_offset((int64_t)c * 8, row, rows, K, 8)) = pack8_fp8(v[i], r);
    }
    if (lane == 0) scales[row] = r.s;
  }
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
    for (int64_t c = lane; c < chunks; c += 64)
      *reinterpret_cast<uint2*>(codes + panel_offset(c * 8, row, rows, K, 8)) = pack8_fp8(src[c], r);
    if (lane == 0) scales[row] = r.s;
  }
}

// ------------------------------------------------------------ launch ------

static int grid_for_rows(int64_t rows) {
  int64_t blocks = (rows + kQuantWaves - 1) / kQuantWaves;
  const int64_t cap = 1 << 16;  // one row per wave up to 2^18 rows; rows loop beyond
  return (int)(blocks < cap ? blocks : cap);
}

template <int B>
static void launch_mxfp4_b(const void* x, int64_t rows, int64_t K, int64_t ld, void* codes, void* scales,
                           hipStream_t s) {
  hipLaunchKernelGGL(mxfp4_quant_kernel<B>, dim3(grid_for_rows(rows)), dim3(64 * kQuantWaves), 0, s,
                     static_cast<const uint16_t*>(x), rows, K, ld, static_cast<uint8_t*>(codes),
                     static_cast<uint32_t*>(scales));
}

hipError_t launch_mxfp4_quant(const void* x, int64_t rows, int64_t K, int64_t ld,
                              void* codes, void* scales, hipStream_t s) {
  // chunks per lane, split into equal batches of at most 16, rounded up to even
  const int64_t per_lane = ((K >> 3) + 63) / 64;
  const int64_t n_batches = (per_lane + 15) / 16;
  const int64_t b = ((per_lane + n_batches - 1) / n_batches + 1) & ~int64_t(1);
  switch (b) {
    case 2: launch_mxfp4_b<2>(x, rows, K, ld, codes, scales, s); break;
    case 4: launch_mxfp4_b<4>(x, rows, K, ld, codes, scales, s); break;
    case 6: launch_mxfp4_b<6>(x, rows, K, ld, codes, scales, s); break;
    case 8: launch_mxfp4_b<8>(x, rows, K, ld, codes, scales, s); break;
    case 10: launch_mxfp4_b<10>(x, rows, K, ld, codes, scales, s); break;
    case 12: launch_mxfp4_b<12>(x, rows, K, ld, codes, scales, s); break;
    case 14: launch_mxfp4_b<14>(x, rows, K, ld, codes, scales, s); break;
    default: launch_mxfp4_b<16>(x, rows, K, ld, codes, scales, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_fp8_quant(const void* x, int64_t rows, int64_t K, int64_t ld,
                            void* codes, void* scales, hipStream_t s) {
  const auto* xs = static_cast<const uint16_t*>(x);
  auto* cs = static_cast<uint8_t*>(codes);
  auto* ss = static_cast<float*>(scales);
  const dim3 grid(grid_for_rows(rows)), block(64 * kQuantWaves);
  // one read per row while the row fits the registers of a wave
  if (K <= 64 * 8 * 4)
    hipLaunchKernelGGL(fp8_quant_row_kernel<4>, grid, block, 0, s, xs, rows, K, ld, cs, ss);
  else if (K <= 64 * 8 * 12)
    hipLaunchKernelGGL(fp8_quant_row_kernel<12>, grid, block, 0, s, xs, rows, K, ld, cs, ss);
  else if (K <= 64 * 8 * 28)
    hipLaunchKernelGGL(fp8_quant_row_kernel<28>, grid, block, 0, s, xs, rows, K, ld, cs, ss);
  else
    hipLaunchKernelGGL(fp8_quant_kernel, grid, block, 0, s, xs, rows, K, ld, cs, ss);
  return hipGetLastError();
}

}  // namespace mxq
