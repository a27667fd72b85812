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

#include <type_traits>

#include "mxq_convert.h"
#include "mxq_device.h"
#include "mxq_internal.h"

namespace mxq {

// ------------------------------------------------------------ MXFP4 -------
//
// MXFP4 codes are stored K-panel-major: K is cut into panels of 128 elements
// (the last one narrower when K % 128 != 0), and panel p holds every row's
// codes of elements 128p .. 128p + w_p - 1 contiguously, row after row (64 B
// per row for a full panel). One GEMM stage of a 256-row tile is then one
// contiguous block. Scales are group-major, [ceil(K/128)][rows][4]: the four
// E8M0 bytes of one row's blocks in one panel form one dword, and the dwords
// of all rows for one panel are contiguous.
//
// Mapping: a wave unit is 16 consecutive rows times up to 4 panels, one row
// per step. Lane l takes 8-element chunk l % 16 of panel l / 16: one load
// reads 1 KiB of one row (512 consecutive elements), four neighbouring lanes
// hold one 32-element block (a quad-shuffle max gives its amax), and one store
// writes the row's 64 code bytes of each of the 4 panels (consecutive rows of
// a panel are adjacent, so the unit's 16 rows fill 1 KiB per panel). All 16
// loads of a unit (16 KiB per wave) are issued before the first conversion.
// (Four rows x 256 B per load, with 256 B code stores, ran as fast at
// K = 5120 and 4-11% slower at K = 3072 and 13824, same bytes.) The block
// amax is a max over the magnitude bit patterns (sign cleared), exact for
// finite bf16, with no float compare and no denormal flush.

constexpr int kQuantWaves = 4;  // waves per workgroup
constexpr int kMxRows = 16;     // rows per wave unit
constexpr int kMxPanels = 4;    // panels per wave unit (fewer in the last one)
constexpr int64_t kStreamInputBytes = int64_t(256) << 20;  // the last-level (Infinity) cache

// 16-byte load of 8 bf16 input elements; with NT, with the non-temporal hint
// (inputs larger than the last-level cache, read once: see mxfp4_quant_kernel).
template <bool NT>
__device__ __forceinline__ uint4 load_chunk(const uint4* p) {
  if constexpr (NT) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(q.x, q.y, q.z, q.w);
  } else {
    return *p;
  }
}

// Max over the 4 lanes of a quad, by DPP quad permutations (lane ^ 1, lane ^ 2).
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  v = umax(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));
  v = umax(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));
  return v;
}

// WEIGHT only names the instance: the offline weight pack and the activation
// quantizer run the same code, and separate symbols keep their launches apart
// in profiles. NT loads the input with the non-temporal hint: an input larger
// than the 256 MiB Infinity Cache is not going to be found there by the next
// pass, and streaming it keeps the codes the GEMM reads next (A14B 720p,
// 774 MB: 212 -> 195 us); a smaller input is, and loses its reuse (TI2V-5B,
// 70 MB: 16.5 -> 17.9 us), so the launch picks by size. Same bytes either way.
template <bool WEIGHT, bool NT>
__global__ __launch_bounds__(64 * kQuantWaves) void mxfp4_quant_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t K, int64_t ld,
    uint8_t* __restrict__ codes, uint32_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t unit0 = (int64_t)blockIdx.x * kQuantWaves + (threadIdx.x >> 6);
  const int64_t n_waves = (int64_t)gridDim.x * kQuantWaves;
  const int64_t chunks = K >> 3;  // 8-element chunks per row
  const int n_panels = (int)((K + 127) >> 7);
  const int pchunks = (n_panels + kMxPanels - 1) / kMxPanels;
  const int64_t units = (rows + kMxRows - 1) / kMxRows * pchunks;
  const int pp = lane >> 4, c = lane & 15;  // panel within the unit, chunk within the panel
  for (int64_t u = unit0; u < units; u += n_waves) {
    const int64_t row0 = u / pchunks * kMxRows;
    const int p = (int)(u % pchunks) * kMxPanels + pp;
    const int64_t ch = 16 * (int64_t)p + c;
    // chunks is a multiple of 4 and a panel's first chunk of 16, so a whole
    // 4-lane block is in or out of range: the shuffles stay uniform per block
    const bool ch_ok = ch < chunks;
    uint4 v[kMxRows];
#pragma unroll
    for (int t = 0; t < kMxRows; ++t) {
      const int64_t row = row0 + t;
      v[t] = row < rows && ch_ok ? load_chunk<NT>(reinterpret_cast<const uint4*>(x + row * ld) + ch)
                                 : make_uint4(0, 0, 0, 0);
    }
    const int64_t w = K - 128 * (int64_t)p < 128 ? K - 128 * (int64_t)p : 128;  // panel width
#pragma unroll
    for (int t = 0; t < kMxRows; ++t) {
      const int64_t row = row0 + t;
      const uint32_t amax = quad_max(chunk_amax(v[t]));
      const uint32_t sb = ch_ok ? mx_scale_byte(amax) : 0u;
      const uint32_t packed = pack8_fp4(v[t], sb);
      // the panel's 4 block scales (block leaders at lanes +0, +4, +8, +12 of
      // the 16-lane row): DPP row shifts left by 4, 8, 12
      const uint32_t s1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)sb, 0x104, 0xF, 0xF, true);
      const uint32_t s2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)sb, 0x108, 0xF, 0xF, true);
      const uint32_t s3 = (uint32_t)__builtin_amdgcn_mov_dpp((int)sb, 0x10C, 0xF, 0xF, true);
      if (row < rows && p < n_panels) {
        if (ch_ok) *reinterpret_cast<uint32_t*>(codes + (int64_t)p * 64 * rows + row * (w >> 1) + 4 * c) = packed;
        if (c == 0) scales[(int64_t)p * rows + row] = sb | (s1 << 8) | (s2 << 16) | (s3 << 24);
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
      if (c < chunks) reinterpret_cast<uint2*>(codes + row * K)[c] = pack8_fp8(v[i], r);
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
    uint2* dst = reinterpret_cast<uint2*>(codes + row * K);
    for (int64_t c = lane; c < chunks; c += 64) dst[c] = pack8_fp8(src[c], r);
    if (lane == 0) scales[row] = r.s;
  }
}

// ---------------------------------------------------- transform_on -------
//
// The transform_on mode keeps a block on W4A4 but rotates the K dimension of
// each linear's input by a fixed block-diagonal Walsh-Hadamard matrix (one
// 128-point block per MXFP4 code panel) and rescales each channel
// (SmoothQuant), the weight offline with the inverse rescale; see section
// "Mixed-Precision selection" of the page. The arithmetic is fp32 in a fixed
// order: butterflies for h = 1, 2, 4 (inside a lane's 8 elements), then
// h = 8, 16, 32, 64 (lanes whose chunk index differs in bit h / 8), each an
// fp32 a + b or a - b; then one fp32 multiply by the channel's factor (which
// holds 1 / sqrt(128)); then rounding to bf16 and the MXFP4 rule above.

constexpr uint32_t kInvSqrt128Bits = 0x3DB504F3u;  // RN(1 / sqrt(128)) in fp32

// 128-point transform of one row panel held by 16 lanes, 8 elements each:
// lane chunk c holds elements 8c .. 8c + 7. Every lane of the wave takes part
// in the exchanges (no lane may be inactive here).
//
// Stages h = 1, 2, 4 run inside the lane. Stages h = 8, 16, 32, 64 pair the
// lanes whose chunk index differs in bit 1, 2, 4, 8 (lane ^ 1, ^ 2, ^ 4, ^ 8
// within the 16-lane row). They keep a known sign per lane: afterwards the
// lane holds (-1)^popcount(c) times the transform (callers fold that sign
// into the channel factor, an exact change). In that form each stage is one
// fused multiply-add of the partner's value, read through DPP, into the
// lane's own: with u = s v (the partner's sign equal to the lane's s before
// the stage), the lane whose bit is clear computes u_p + u = s (a + b) and
// keeps its sign, the other computes u - u_p = -s (a - b) and flips it. Each
// is one rounding of a + b or a - b, up to that sign; only the sign of an
// exact zero is lost, and callers turn every exact zero into +0.
// The DPP patterns: lane ^ 1 and ^ 2 are quad permutations, ^ 8 the row
// rotation by 8, ^ 4 the half-row mirror (lane ^ 7) then the quad
// permutation lane ^ 3. All are their own inverses, so no direction
// convention matters. A DPP read of a register needs two wait states after
// a VALU write of it: the block opens with them, and inside it every DPP
// source was written eight instructions earlier.
__device__ __forceinline__ void fwht128_lanes(float (&f)[8], int c) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if ((e & h) == 0) {
        const float a = f[e], b = f[e + h];
        f[e] = a + b;
        f[e + h] = a - b;
      }
  const float s1 = (c & 1) ? -1.0f : 1.0f, s2 = (c & 2) ? -1.0f : 1.0f;
  const float s4 = (c & 4) ? -1.0f : 1.0f, s8 = (c & 8) ? -1.0f : 1.0f;
  float t0, t1, t2, t3, t4, t5, t6, t7;
#define MXQ_DPP_FMAC(D, S, SG, PAT) "v_fmac_f32_dpp " D ", " S ", " SG " " PAT " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
#define MXQ_DPP_MOV(D, S, PAT) "v_mov_b32_dpp " D ", " S " " PAT " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
#define MXQ_STAGE8(SG, PAT)                                                                                   \
  MXQ_DPP_FMAC("%0", "%0", SG, PAT) MXQ_DPP_FMAC("%1", "%1", SG, PAT) MXQ_DPP_FMAC("%2", "%2", SG, PAT)      \
  MXQ_DPP_FMAC("%3", "%3", SG, PAT) MXQ_DPP_FMAC("%4", "%4", SG, PAT) MXQ_DPP_FMAC("%5", "%5", SG, PAT)      \
  MXQ_DPP_FMAC("%6", "%6", SG, PAT) MXQ_DPP_FMAC("%7", "%7", SG, PAT)
  asm volatile(
      "s_nop 1\n\t"
      MXQ_STAGE8("%16", "quad_perm:[1,0,3,2]")
      MXQ_STAGE8("%17", "quad_perm:[2,3,0,1]")
      MXQ_DPP_MOV("%8", "%0", "row_half_mirror") MXQ_DPP_MOV("%9", "%1", "row_half_mirror")
      MXQ_DPP_MOV("%10", "%2", "row_half_mirror") MXQ_DPP_MOV("%11", "%3", "row_half_mirror")
      MXQ_DPP_MOV("%12", "%4", "row_half_mirror") MXQ_DPP_MOV("%13", "%5", "row_half_mirror")
      MXQ_DPP_MOV("%14", "%6", "row_half_mirror") MXQ_DPP_MOV("%15", "%7", "row_half_mirror")
      MXQ_DPP_FMAC("%0", "%8", "%18", "quad_perm:[3,2,1,0]") MXQ_DPP_FMAC("%1", "%9", "%18", "quad_perm:[3,2,1,0]")
      MXQ_DPP_FMAC("%2", "%10", "%18", "quad_perm:[3,2,1,0]") MXQ_DPP_FMAC("%3", "%11", "%18", "quad_perm:[3,2,1,0]")
      MXQ_DPP_FMAC("%4", "%12", "%18", "quad_perm:[3,2,1,0]") MXQ_DPP_FMAC("%5", "%13", "%18", "quad_perm:[3,2,1,0]")
      MXQ_DPP_FMAC("%6", "%14", "%18", "quad_perm:[3,2,1,0]") MXQ_DPP_FMAC("%7", "%15", "%18", "quad_perm:[3,2,1,0]")
      MXQ_STAGE8("%19", "row_ror:8")
      : "+v"(f[0]), "+v"(f[1]), "+v"(f[2]), "+v"(f[3]), "+v"(f[4]), "+v"(f[5]), "+v"(f[6]), "+v"(f[7]),
        "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3), "=&v"(t4), "=&v"(t5), "=&v"(t6), "=&v"(t7)
      : "v"(s1), "v"(s2), "v"(s4), "v"(s8));
#undef MXQ_STAGE8
#undef MXQ_DPP_MOV
#undef MXQ_DPP_FMAC
}

__device__ __forceinline__ void bf16x8_to_f32(const uint4 v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = as_float(w[i] << 16);
    f[2 * i + 1] = as_float(w[i] & 0xFFFF0000u);
  }
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  const f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// The MXFP4 quantizer's mapping and stores, on transformed rows: each step's
// 16 lanes of a row panel transform their 128 elements together, apply the
// channel factors as RN(t * mult + 0), round to bf16, and continue exactly as
// the plain quantizer. A lane keeps its panel for the whole unit, so it reads
// its 8 channel factors once. K is a multiple of 128 (whole panels). NT: the
// non-temporal input loads of the plain quantizer, for the same reason and
// chosen by the same size rule.
template <bool NT>
__global__ __launch_bounds__(64 * kQuantWaves) void mxfp4_hadamard_quant_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t K, int64_t ld, const float* __restrict__ mult,
    uint8_t* __restrict__ codes, uint32_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t unit0 = (int64_t)blockIdx.x * kQuantWaves + (threadIdx.x >> 6);
  const int64_t n_waves = (int64_t)gridDim.x * kQuantWaves;
  const int n_panels = (int)(K >> 7);
  const int pchunks = (n_panels + kMxPanels - 1) / kMxPanels;
  const int64_t units = (rows + kMxRows - 1) / kMxRows * pchunks;
  const int pp = lane >> 4, c = lane & 15;  // panel within the unit, chunk within the panel
  for (int64_t u = unit0; u < units; u += n_waves) {
    const int64_t row0 = u / pchunks * kMxRows;
    const int p = (int)(u % pchunks) * kMxPanels + pp;
    const bool p_ok = p < n_panels;
    uint4 v[kMxRows];
#pragma unroll
    for (int t = 0; t < kMxRows; ++t) {
      const int64_t row = row0 + t;
      v[t] = row < rows && p_ok ? load_chunk<NT>(reinterpret_cast<const uint4*>(x + row * ld) + 16 * (int64_t)p + c)
                                : make_uint4(0, 0, 0, 0);
    }
    // the factors with the lane's sign from the transform folded in
    float m[8];
    if (p_ok) {
      const uint32_t neg = (uint32_t)(__builtin_popcount(c) & 1) << 31;
      const float4 m0 = reinterpret_cast<const float4*>(mult + 128 * (int64_t)p + 8 * c)[0];
      const float4 m1 = reinterpret_cast<const float4*>(mult + 128 * (int64_t)p + 8 * c)[1];
      m[0] = m0.x; m[1] = m0.y; m[2] = m0.z; m[3] = m0.w;
      m[4] = m1.x; m[5] = m1.y; m[6] = m1.z; m[7] = m1.w;
#pragma unroll
      for (int e = 0; e < 8; ++e) m[e] = as_float(as_uint(m[e]) ^ neg);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) m[e] = 0.0f;
    }
#pragma unroll
    for (int t = 0; t < kMxRows; ++t) {
      const int64_t row = row0 + t;
      float f[8];
      bf16x8_to_f32(v[t], f);
      fwht128_lanes(f, c);
      // RN(t * mult + 0): exact zeros become +0 (their sign is not known here)
      float q[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) q[e] = __builtin_fmaf(f[e], m[e], 0.0f);
      uint4 tv;
      tv.x = bf16x2_rne(q[0], q[1]);
      tv.y = bf16x2_rne(q[2], q[3]);
      tv.z = bf16x2_rne(q[4], q[5]);
      tv.w = bf16x2_rne(q[6], q[7]);
      const uint32_t amax = quad_max(chunk_amax(tv));
      const uint32_t sb = mx_scale_byte(amax);
      const uint32_t packed = pack8_fp4(tv, sb);
      const uint32_t s1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)sb, 0x104, 0xF, 0xF, true);
      const uint32_t s2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)sb, 0x108, 0xF, 0xF, true);
      const uint32_t s3 = (uint32_t)__builtin_amdgcn_mov_dpp((int)sb, 0x10C, 0xF, 0xF, true);
      if (row < rows && p_ok) {
        *reinterpret_cast<uint32_t*>(codes + (int64_t)p * 64 * rows + row * 64 + 4 * c) = packed;
        if (c == 0) scales[(int64_t)p * rows + row] = sb | (s1 << 8) | (s2 << 16) | (s3 << 24);
      }
    }
  }
}

// Calibration for SmoothQuant: per-channel max |transform(x)| (unnormalized
// butterflies, no factor) over the rows, folded into a running maximum
// amax[K] (fp32 bit patterns, non-negative: unsigned atomic max). Workgroup
// (panel p, row split): its 4 waves take 4 rows per step each; lane chunk c
// keeps the maxima of channels 128p + 8c .. + 7; one atomic per channel per
// workgroup.
constexpr int kAmaxRowsUnroll = 4;

__global__ __launch_bounds__(64 * kQuantWaves) void hadamard_amax_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t K, int64_t ld, int64_t rows_per_split,
    uint32_t* __restrict__ amax_bits) {
  __shared__ uint32_t red[kQuantWaves][128];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rs = lane >> 4, c = lane & 15;
  const int p = blockIdx.x;
  const int64_t r_begin = (int64_t)blockIdx.y * rows_per_split;
  const int64_t r_end = r_begin + rows_per_split < rows ? r_begin + rows_per_split : rows;
  uint32_t m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  constexpr int STEP = 4 * kQuantWaves;  // rows per workgroup step
  for (int64_t r0 = r_begin + 4 * wave; r0 < r_end; r0 += STEP * kAmaxRowsUnroll) {
    uint4 v[kAmaxRowsUnroll];
#pragma unroll
    for (int i = 0; i < kAmaxRowsUnroll; ++i) {
      const int64_t row = r0 + STEP * i + rs;
      v[i] = row < r_end ? reinterpret_cast<const uint4*>(x + row * ld)[16 * (int64_t)p + c] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kAmaxRowsUnroll; ++i) {
      float f[8];
      bf16x8_to_f32(v[i], f);
      fwht128_lanes(f, c);
#pragma unroll
      for (int e = 0; e < 8; ++e) m[e] = umax(m[e], as_uint(f[e]) & 0x7FFFFFFFu);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    m[e] = umax(m[e], (uint32_t)__shfl_xor((int)m[e], 16));
    m[e] = umax(m[e], (uint32_t)__shfl_xor((int)m[e], 32));
  }
  if (rs == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) red[wave][8 * c + e] = m[e];
  }
  __syncthreads();
  if (threadIdx.x < 128) {
    uint32_t b = red[0][threadIdx.x];
#pragma unroll
    for (int w = 1; w < kQuantWaves; ++w) b = umax(b, red[w][threadIdx.x]);
    if (b != 0) atomicMax(amax_bits + 128 * (int64_t)p + threadIdx.x, b);
  }
}

// SmoothQuant factors at migration strength 0.5: lambda = sqrt(ax / aw) (1
// where either maximum is 0), act_mult = RN(RN(1 / lambda) / sqrt(128)),
// w_mult = RN(lambda / sqrt(128)), with 1 / sqrt(128) the fp32 constant above
// (IEEE division and square root).
__global__ void smoothquant_factor_kernel(const float* __restrict__ ax, const float* __restrict__ aw, int64_t K,
                                          float* __restrict__ act_mult, float* __restrict__ w_mult) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (k >= K) return;
  const float a = ax[k], w = aw[k];
  const float lam = (a > 0.0f && w > 0.0f) ? __builtin_sqrtf(a / w) : 1.0f;
  const float c0 = as_float(kInvSqrt128Bits);
  const float inv = 1.0f / lam;
  act_mult[k] = inv * c0;
  w_mult[k] = lam * c0;
}

// ------------------------------------------------------ FP8 static -------
//
// Static (per-tensor) FP8: one scale s = amax / 448 for the whole tensor,
// from an amax gathered beforehand over calibration data. The quantizer needs
// no reduction: each lane turns 8 elements (16 bytes read) into 8 codes (8
// bytes written), and every row's scale slot gets s, so the W4A8 GEMM takes
// the result as it takes per-token activations. Quotients beyond 448
// saturate (a static scale can be exceeded at run time).

__device__ __forceinline__ float fp8_static_signed_quotient(uint32_t bits16, const Fp8Row& r) {
  const float q = r.s == 0.0f ? 0.0f : fp8_static_quotient(as_float((bits16 & 0x7FFFu) << 16), r);
  return as_float(as_uint(q) | ((bits16 & 0x8000u) << 16));
}

__device__ __forceinline__ uint2 pack8_fp8_static(const uint4 c, const Fp8Row& r) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  uint32_t out[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float q0 = fp8_static_signed_quotient(w[2 * i] & 0xFFFFu, r);
    const float q1 = fp8_static_signed_quotient(w[2 * i] >> 16, r);
    const float q2 = fp8_static_signed_quotient(w[2 * i + 1] & 0xFFFFu, r);
    const float q3 = fp8_static_signed_quotient(w[2 * i + 1] >> 16, r);
    uint32_t o = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
    o = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, (int)o, true);
    out[i] = o;
  }
  return make_uint2(out[0], out[1]);
}

constexpr int kStaticUnroll = 4;  // 16-byte loads in flight per lane

// One wave per row (rows loop beyond the grid); lanes walk the row's 8-element
// chunks, kStaticUnroll loads ahead of the conversions.
__global__ __launch_bounds__(64 * kQuantWaves) void fp8_static_quant_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t K, int64_t ld, const float* __restrict__ amax,
    uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t wave_id = (int64_t)blockIdx.x * kQuantWaves + (threadIdx.x >> 6);
  const int64_t n_waves = (int64_t)gridDim.x * kQuantWaves;
  const int64_t chunks = K >> 3;
  const Fp8Row r = fp8_scale_setup(*amax);
  for (int64_t row = wave_id; row < rows; row += n_waves) {
    const uint4* src = reinterpret_cast<const uint4*>(x + row * ld);
    uint2* dst = reinterpret_cast<uint2*>(codes + row * K);
    for (int64_t c0 = lane; c0 < chunks; c0 += 64 * kStaticUnroll) {
      uint4 v[kStaticUnroll];
#pragma unroll
      for (int i = 0; i < kStaticUnroll; ++i) {
        const int64_t c = c0 + 64 * i;
        v[i] = c < chunks ? src[c] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < kStaticUnroll; ++i) {
        const int64_t c = c0 + 64 * i;
        if (c < chunks) dst[c] = pack8_fp8_static(v[i], r);
      }
    }
    if (lane == 0) scales[row] = r.s;
  }
}

// Calibration: largest |x| of a [rows, K] bf16 matrix, folded into a running
// maximum. Magnitude bit patterns order like the values (finite inputs), and
// a bf16 pattern shifted left by 16 is the fp32 pattern of the same value, so
// the running maximum is an fp32 updated with an unsigned atomic max (max is
// order-free: the result does not depend on the schedule). Each wave keeps a
// maximum over its rows; one atomic per workgroup.
__global__ __launch_bounds__(64 * kQuantWaves) void fp8_amax_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t K, int64_t ld, uint32_t* __restrict__ amax_bits) {
  __shared__ uint32_t wave_max_lds[kQuantWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t wave_id = (int64_t)blockIdx.x * kQuantWaves + wave;
  const int64_t n_waves = (int64_t)gridDim.x * kQuantWaves;
  const int64_t chunks = K >> 3;
  uint32_t m = 0;
  for (int64_t row = wave_id; row < rows; row += n_waves) {
    const uint4* src = reinterpret_cast<const uint4*>(x + row * ld);
    for (int64_t c0 = lane; c0 < chunks; c0 += 64 * kStaticUnroll) {
      uint4 v[kStaticUnroll];
#pragma unroll
      for (int i = 0; i < kStaticUnroll; ++i) {
        const int64_t c = c0 + 64 * i;
        v[i] = c < chunks ? src[c] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < kStaticUnroll; ++i) m = umax(m, chunk_amax(v[i]));
    }
  }
  m = wave_max(m);
  if (lane == 0) wave_max_lds[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t b = wave_max_lds[0];
#pragma unroll
    for (int w = 1; w < kQuantWaves; ++w) b = umax(b, wave_max_lds[w]);
    if (b != 0) atomicMax(amax_bits, b << 16);
  }
}

// ------------------------------------------------------------ launch ------

static int grid_for_rows(int64_t rows) {
  int64_t blocks = (rows + kQuantWaves - 1) / kQuantWaves;
  const int64_t cap = 1 << 16;  // one row per wave up to 2^18 rows; rows loop beyond
  return (int)(blocks < cap ? blocks : cap);
}

hipError_t launch_mxfp4_quant(const void* x, int64_t rows, int64_t K, int64_t ld,
                              void* codes, void* scales, hipStream_t s, bool weight) {
  const int64_t pchunks = ((K + 127) / 128 + kMxPanels - 1) / kMxPanels;
  const int64_t units = (rows + kMxRows - 1) / kMxRows * pchunks;
  int64_t blocks = (units + kQuantWaves - 1) / kQuantWaves;
  if (blocks > (1 << 16)) blocks = 1 << 16;  // units loop beyond
  const auto* xs = static_cast<const uint16_t*>(x);
  auto* cs = static_cast<uint8_t*>(codes);
  auto* ss = static_cast<uint32_t*>(scales);
  const dim3 grid((unsigned)blocks), block(64 * kQuantWaves);
  const bool streamed = rows * ld * 2 > kStreamInputBytes;
  if (weight)
    hipLaunchKernelGGL((mxfp4_quant_kernel<true, false>), grid, block, 0, s, xs, rows, K, ld, cs, ss);
  else if (streamed)
    hipLaunchKernelGGL((mxfp4_quant_kernel<false, true>), grid, block, 0, s, xs, rows, K, ld, cs, ss);
  else
    hipLaunchKernelGGL((mxfp4_quant_kernel<false, false>), grid, block, 0, s, xs, rows, K, ld, cs, ss);
  return hipGetLastError();
}

hipError_t launch_fp8_quant(const void* x, int64_t rows, int64_t K, int64_t ld,
                            void* codes, void* scales, hipStream_t s) {
  const auto* xs = static_cast<const uint16_t*>(x);
  auto* cs = static_cast<uint8_t*>(codes);
  auto* ss = static_cast<float*>(scales);
  const dim3 grid(grid_for_rows(rows)), block(64 * kQuantWaves);
  // one read per row while the row fits the registers of a wave (the
  // non-temporal input hint of the MXFP4 quantizer made the W4A8 GEMM that
  // follows slower by as much as it saved here, so these loads keep the default)
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

hipError_t launch_mxfp4_hadamard_quant(const void* x, int64_t rows, int64_t K, int64_t ld, const float* mult,
                                       void* codes, void* scales, hipStream_t s) {
  const int64_t pchunks = (K / 128 + kMxPanels - 1) / kMxPanels;
  const int64_t units = (rows + kMxRows - 1) / kMxRows * pchunks;
  int64_t blocks = (units + kQuantWaves - 1) / kQuantWaves;
  if (blocks > (1 << 16)) blocks = 1 << 16;  // units loop beyond
  if (rows * ld * 2 > kStreamInputBytes)
    hipLaunchKernelGGL(mxfp4_hadamard_quant_kernel<true>, dim3((unsigned)blocks), dim3(64 * kQuantWaves), 0, s,
                       static_cast<const uint16_t*>(x), rows, K, ld, mult, static_cast<uint8_t*>(codes),
                       static_cast<uint32_t*>(scales));
  else
    hipLaunchKernelGGL(mxfp4_hadamard_quant_kernel<false>, dim3((unsigned)blocks), dim3(64 * kQuantWaves), 0, s,
                       static_cast<const uint16_t*>(x), rows, K, ld, mult, static_cast<uint8_t*>(codes),
                       static_cast<uint32_t*>(scales));
  return hipGetLastError();
}

hipError_t launch_hadamard_amax(const void* x, int64_t rows, int64_t K, int64_t ld, float* amax, hipStream_t s) {
  const int64_t panels = K / 128;
  const int64_t step = 4 * kQuantWaves;
  // about 2048 workgroups in all; each split a multiple of the workgroup step
  int64_t splits = (2048 + panels - 1) / panels;
  const int64_t max_splits = (rows + step - 1) / step;
  splits = splits < max_splits ? splits : max_splits;
  splits = splits > 0 ? splits : 1;
  int64_t per = (rows + splits - 1) / splits;
  per = (per + step - 1) / step * step;
  splits = (rows + per - 1) / per;
  hipLaunchKernelGGL(hadamard_amax_kernel, dim3((unsigned)panels, (unsigned)splits), dim3(64 * kQuantWaves), 0, s,
                     static_cast<const uint16_t*>(x), rows, K, ld, per, reinterpret_cast<uint32_t*>(amax));
  return hipGetLastError();
}

hipError_t launch_smoothquant_factors(const float* act_amax, const float* w_amax, int64_t K, float* act_mult,
                                      float* w_mult, hipStream_t s) {
  hipLaunchKernelGGL(smoothquant_factor_kernel, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, s, act_amax,
                     w_amax, K, act_mult, w_mult);
  return hipGetLastError();
}

// Static FP8 and calibration grids: a few workgroups per CU, rows loop.
static int grid_for_static(int64_t rows) {
  const int64_t blocks = (rows + kQuantWaves - 1) / kQuantWaves;
  const int64_t cap = 4096;
  return (int)(blocks < cap ? (blocks > 0 ? blocks : 1) : cap);
}

hipError_t launch_fp8_static_quant(const void* x, int64_t rows, int64_t K, int64_t ld, const float* amax,
                                   void* codes, void* scales, hipStream_t s) {
  hipLaunchKernelGGL(fp8_static_quant_kernel, dim3(grid_for_static(rows)), dim3(64 * kQuantWaves), 0, s,
                     static_cast<const uint16_t*>(x), rows, K, ld, amax, static_cast<uint8_t*>(codes),
                     static_cast<float*>(scales));
  return hipGetLastError();
}

hipError_t launch_fp8_amax(const void* x, int64_t rows, int64_t K, int64_t ld, float* amax, hipStream_t s) {
  const int64_t cap = 1024;  // workgroups: one atomic each
  int64_t blocks = (rows + kQuantWaves - 1) / kQuantWaves;
  blocks = blocks < cap ? blocks : cap;
  hipLaunchKernelGGL(fp8_amax_kernel, dim3((unsigned)blocks), dim3(64 * kQuantWaves), 0, s,
                     static_cast<const uint16_t*>(x), rows, K, ld, reinterpret_cast<uint32_t*>(amax));
  return hipGetLastError();
}

}  // namespace mxq
