// mxq_gemm.hip - scaled-MFMA GEMM on MXFP4 weights and MXFP4 / FP8
// activations for gfx950.
//
// Computes y[m][n] = epi( sum_k deqA[m][k] * deqW[n][k] + bias[n] ) with fp32
// accumulation and a bf16 result: the native execution of W4A4 (FP4 x FP4,
// E8M0 scales on both sides) and W4A8 (FP8 x FP4, per-token fp32 scale applied
// to the fp32 sum) of section "Quantization formats" of the page "Quark
// Mixed-Precision Quantization for Wan2.2 Video Generation on AMD Instinct
// GPUs".
//
// Instruction: v_mfma_scale_f32_32x32x64_f8f6f4. Each lane feeds one 32-element
// K block of one row of each operand (lane l: row l % 32, block slot l / 32),
// plus that block's E8M0 scale byte, picked out of a 32-bit register by the
// instruction's op_sel. The product is transposed on purpose: the weight is
// the instruction's first operand (rows = n) and the activation the second
// (columns = m), so a lane's accumulators hold 4 consecutive n of one token m
// and the bf16 result leaves in 8-byte stores.
//
// K order inside a 256-element tile (8 blocks): lane slot g (0/1) owns blocks
// 4g .. 4g+3, and MFMA step kk (0..3) consumes block 4g + kk from both
// operands. A lane's data for a tile is then 64 contiguous bytes (FP4) or
// 128 (FP8) and its 4 scale bytes are contiguous too (op_sel = kk). The sum
// over K is the same set of products as in natural order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq_convert.h"
#include "mxq_internal.h"

namespace mxq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kFmtFp8 = 0;  // cbsz / blgp format code: FP8 E4M3
constexpr int kFmtFp4 = 4;  // cbsz / blgp format code: FP4 E2M1
constexpr uint32_t kUnitScales = 0x7F7F7F7Fu;  // four E8M0 bytes of 2^0

struct FragFp4 {  // one lane, one K tile: 4 blocks of 16 bytes + 4 scale bytes
  uint4 d[4];
  uint32_t sc;
};
struct FragFp8 {  // one lane, one K tile: 4 blocks of 32 bytes
  uint4 d[8];
};

__device__ __forceinline__ uint32_t load_scales4(const uint8_t* p, int b0, int KB, bool tail) {
  uint32_t s = 0;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    uint32_t v = (!tail || b0 + t < KB) ? (uint32_t)p[b0 + t] : 0u;
    s |= v << (8 * t);
  }
  return s;
}

template <bool TAIL>
__device__ __forceinline__ void load_fp4(FragFp4& f, const uint8_t* q, const uint8_t* sc, int b0, int KB) {
  const uint4* p = reinterpret_cast<const uint4*>(q) + b0;
#pragma unroll
  for (int t = 0; t < 4; ++t) f.d[t] = (!TAIL || b0 + t < KB) ? p[t] : make_uint4(0, 0, 0, 0);
  f.sc = load_scales4(sc, b0, KB, TAIL);
}

template <bool TAIL>
__device__ __forceinline__ void load_fp8(FragFp8& f, const uint8_t* q, int b0, int KB) {
  const uint4* p = reinterpret_cast<const uint4*>(q) + 2 * b0;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const bool ok = !TAIL || b0 + t < KB;
    f.d[2 * t] = ok ? p[2 * t] : make_uint4(0, 0, 0, 0);
    f.d[2 * t + 1] = ok ? p[2 * t + 1] : make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ v8i op_fp4(const uint4 d) {
  v8i v = {(int)d.x, (int)d.y, (int)d.z, (int)d.w, 0, 0, 0, 0};
  return v;
}
__device__ __forceinline__ v8i op_fp8(const uint4 lo, const uint4 hi) {
  v8i v = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  return v;
}

// One MFMA step kk of a tile for a TN x TM grid of 32x32 accumulators.
template <int MODE, int TN, int TM, int KK, typename XFrag>
__device__ __forceinline__ void mfma_step(v16f (&acc)[TN][TM], const FragFp4 (&wf)[TN],
                                          const XFrag (&xf)[TM], const uint32_t (&xs)[TM]) {
#pragma unroll
  for (int i = 0; i < TN; ++i) {
    const v8i a = op_fp4(wf[i].d[KK]);
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      v8i b;
      if constexpr (MODE == 0) {
        b = op_fp4(reinterpret_cast<const FragFp4&>(xf[j]).d[KK]);
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            a, b, acc[i][j], kFmtFp4, kFmtFp4, KK, (int)wf[i].sc, KK, (int)xs[j]);
      } else {
        const FragFp8& x8 = reinterpret_cast<const FragFp8&>(xf[j]);
        b = op_fp8(x8.d[2 * KK], x8.d[2 * KK + 1]);
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            a, b, acc[i][j], kFmtFp4, kFmtFp8, KK, (int)wf[i].sc, KK, (int)kUnitScales);
      }
    }
  }
}

// Correctness-first kernel: every lane loads its operand fragments straight
// from global memory (L2-served), a wave computes (32 TN) x (32 TM) outputs,
// a workgroup of 4 waves (2 x 2) computes (64 TN) x (64 TM).
template <int MODE, int TN, int TM>
__global__ __launch_bounds__(256) void gemm_direct_kernel(
    const uint8_t* __restrict__ wq, const uint8_t* __restrict__ ws,
    const uint8_t* __restrict__ aq, const void* __restrict__ asc,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y,
    int M, int N, int K, int epi) {
  using XFrag = typename std::conditional<MODE == 0, FragFp4, FragFp8>::type;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 31;
  const int g = lane >> 5;
  const int n0 = blockIdx.x * (64 * TN) + (wave & 1) * (32 * TN);
  const int m0 = blockIdx.y * (64 * TM) + (wave >> 1) * (32 * TM);
  const int KB = K >> 5;
  const int64_t a_row_bytes = MODE == 0 ? (K >> 1) : K;

  const uint8_t* wrow[TN];
  const uint8_t* wsrow[TN];
#pragma unroll
  for (int i = 0; i < TN; ++i) {
    int n = min(n0 + 32 * i + r, N - 1);  // rows past the edge re-read the last row
    wrow[i] = wq + (int64_t)n * (K >> 1);
    wsrow[i] = ws + (int64_t)n * KB;
  }
  const uint8_t* xrow[TM];
  const uint8_t* xsrow[TM];
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    int m = min(m0 + 32 * j + r, M - 1);
    xrow[j] = aq + (int64_t)m * a_row_bytes;
    xsrow[j] = MODE == 0 ? static_cast<const uint8_t*>(asc) + (int64_t)m * KB : nullptr;
  }

  v16f acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  auto tile = [&](int kt, auto tail_tag) {
    constexpr bool TAIL = decltype(tail_tag)::value;
    const int b0 = kt * 8 + 4 * g;
    FragFp4 wf[TN];
    XFrag xf[TM];
    uint32_t xs[TM];
#pragma unroll
    for (int i = 0; i < TN; ++i) load_fp4<TAIL>(wf[i], wrow[i], wsrow[i], b0, KB);
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      if constexpr (MODE == 0) {
        load_fp4<TAIL>(reinterpret_cast<FragFp4&>(xf[j]), xrow[j], xsrow[j], b0, KB);
        xs[j] = reinterpret_cast<FragFp4&>(xf[j]).sc;
      } else {
        load_fp8<TAIL>(reinterpret_cast<FragFp8&>(xf[j]), xrow[j], b0, KB);
        xs[j] = kUnitScales;
      }
    }
    mfma_step<MODE, TN, TM, 0>(acc, wf, xf, xs);
    mfma_step<MODE, TN, TM, 1>(acc, wf, xf, xs);
    mfma_step<MODE, TN, TM, 2>(acc, wf, xf, xs);
    mfma_step<MODE, TN, TM, 3>(acc, wf, xf, xs);
  };

  const int full = KB >> 3;
  for (int kt = 0; kt < full; ++kt) tile(kt, std::false_type{});
  if (KB & 7) tile(full, std::true_type{});

  // Epilogue. Accumulator q of lane (r, g) in a 32x32 tile holds
  // n = 8 (q / 4) + 4 g + (q % 4), m = r.
  const float* tok_scale = static_cast<const float*>(asc);
  const bool vec_store = (N & 3) == 0;
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int m = m0 + 32 * j + r;
    if (m >= M) continue;
    const float sm = MODE == 1 ? tok_scale[m] : 1.0f;
    uint16_t* yrow = y + (int64_t)m * N;
#pragma unroll
    for (int i = 0; i < TN; ++i) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int nb = n0 + 32 * i + 8 * qq + 4 * g;
        uint32_t h[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          float v = acc[i][j][4 * qq + t] * sm;
          if (bias != nullptr && nb + t < N) v += as_float((uint32_t)bias[nb + t] << 16);
          if (epi == 1) v = gelu_tanh(v);
          h[t] = bf16_rne(v);
        }
        if (vec_store && nb + 3 < N) {
          *reinterpret_cast<uint2*>(yrow + nb) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (nb + t < N) yrow[nb + t] = (uint16_t)h[t];
        }
      }
    }
  }
}

template <int MODE, int TN, int TM>
static hipError_t launch_direct(const void* aq, const void* as, const void* wq, const void* ws,
                                const void* bias, int epi, void* y, int64_t M, int64_t N,
                                int64_t K, hipStream_t s) {
  dim3 grid((unsigned)((N + 64 * TN - 1) / (64 * TN)), (unsigned)((M + 64 * TM - 1) / (64 * TM)));
  hipLaunchKernelGGL((gemm_direct_kernel<MODE, TN, TM>), grid, dim3(256), 0, s,
                     static_cast<const uint8_t*>(wq), static_cast<const uint8_t*>(ws),
                     static_cast<const uint8_t*>(aq), as, static_cast<const uint16_t*>(bias),
                     static_cast<uint16_t*>(y), (int)M, (int)N, (int)K, epi);
  return hipGetLastError();
}

hipError_t launch_gemm(int mode, const void* a_codes, const void* a_scales,
                       const void* w_codes, const void* w_scales, const void* bias,
                       int epilogue, void* y, int64_t M, int64_t N, int64_t K,
                       hipStream_t s) {
  if (mode == 0)
    return launch_direct<0, 2, 2>(a_codes, a_scales, w_codes, w_scales, bias, epilogue, y, M, N, K, s);
  return launch_direct<1, 2, 2>(a_codes, a_scales, w_codes, w_scales, bias, epilogue, y, M, N, K, s);
}

const char* gemm_variant_name(int mode, int64_t, int64_t, int64_t) {
  return mode == 0 ? "direct_w4a4_32x32x64_wave64x64_wg128x128"
                   : "direct_w4a8_32x32x64_wave64x64_wg128x128";
}

}  // namespace mxq
