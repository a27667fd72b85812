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
#include <stdlib.h>

#include <array>

#include "mxq_convert.h"
#include "mxq_device.h"
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
struct FragFp8 {  // one lane, one K tile: 4 steps x two 16-byte halves
  uint4 d[8];
};

// MXFP4 codes are K-panel-major: panel p (elements 128p .. 128p + 127, fewer
// in a ragged last panel) holds every row's codes of that range contiguously.
// The codes of panel p of `row` start at byte p * 64 * rows + row * w_p / 2,
// w_p the panel's width (the helper also takes other code widths in bits).
__device__ __forceinline__ const uint8_t* panel_row(const uint8_t* q, int p, int row, int64_t rows, int K,
                                                    int bits) {
  const int w = K - 128 * p < 128 ? K - 128 * p : 128;
  return q + (((int64_t)p * 128 * rows + (int64_t)row * (w > 0 ? w : 0)) * bits >> 3);
}

// Scales are group-major: the dword of group gi (blocks 4gi .. 4gi+3) of row
// `row` sits at sc[gi * rows + row]. A lane slot's four blocks of a 256-wide
// tile are exactly one group (= one code panel), so one dword load serves 4
// MFMA steps.
template <bool TAIL>
__device__ __forceinline__ void load_fp4(FragFp4& f, const uint8_t* q, const uint32_t* sc, int64_t rows, int row,
                                         int gi, int n_groups, int b0, int KB, int K) {
  const uint4* p = reinterpret_cast<const uint4*>(panel_row(q, gi, row, rows, K, 4));
#pragma unroll
  for (int t = 0; t < 4; ++t) f.d[t] = (!TAIL || b0 + t < KB) ? p[t] : make_uint4(0, 0, 0, 0);
  f.sc = (!TAIL || gi < n_groups) ? sc[(int64_t)gi * rows + row] : 0u;
}

// FP8 operand of the mixed FP8 x FP4 instruction. The FP4 operand's lane slot
// h (lanes 32h .. 32h+31) covers K 32h .. 32h+31 of a step in natural nibble
// order, but the FP8 operand is split by halves: its bytes 0..15 in slot h
// pair with K 16h .. 16h+15 and bytes 16..31 with K 32+16h .. 32+16h+15.
// With block kk on FP4 slot 0 and block 4+kk on FP4 slot 1 (see above), FP8
// slot h therefore carries half h of block kk, then half h of block 4+kk.
// FP8 codes are row-major [rows][K].
template <bool TAIL>
__device__ __forceinline__ void load_fp8(FragFp8& f, const uint8_t* q, int row, int kt, int h, int KB, int K) {
  const uint4* p = reinterpret_cast<const uint4*>(q + (int64_t)row * K);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int b0 = kt * 8 + t;
    const int b1 = kt * 8 + 4 + t;
    f.d[2 * t] = (!TAIL || b0 < KB) ? p[2 * b0 + h] : make_uint4(0, 0, 0, 0);
    f.d[2 * t + 1] = (!TAIL || b1 < KB) ? p[2 * b1 + h] : make_uint4(0, 0, 0, 0);
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

  const int n_groups = (KB + 3) >> 2;
  const uint32_t* wsc = reinterpret_cast<const uint32_t*>(ws);
  const uint32_t* xsc = static_cast<const uint32_t*>(asc);
  int wn_row[TN];
#pragma unroll
  for (int i = 0; i < TN; ++i) wn_row[i] = min(n0 + 32 * i + r, N - 1);  // rows past the edge re-read the last row
  int xm_row[TM];
#pragma unroll
  for (int j = 0; j < TM; ++j) xm_row[j] = min(m0 + 32 * j + r, M - 1);

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
    const int gi = kt * 2 + g;
    FragFp4 wf[TN];
    XFrag xf[TM];
    uint32_t xs[TM];
#pragma unroll
    for (int i = 0; i < TN; ++i) load_fp4<TAIL>(wf[i], wq, wsc, N, wn_row[i], gi, n_groups, b0, KB, K);
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      if constexpr (MODE == 0) {
        load_fp4<TAIL>(reinterpret_cast<FragFp4&>(xf[j]), aq, xsc, M, xm_row[j], gi, n_groups, b0, KB, K);
        xs[j] = reinterpret_cast<FragFp4&>(xf[j]).sc;
      } else {
        load_fp8<TAIL>(reinterpret_cast<FragFp8&>(xf[j]), aq, xm_row[j], kt, g, KB, K);
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

// ---------------------------------------------------------------------------
// LDS-pipelined persistent kernel for the large shapes.
//
// Workgroup tile 256 (n) x 256 (m), 4 waves in a 2 x 2 grid, each wave owns a
// 128 x 128 output block = 4 x 4 MFMA tiles (256 fp32 accumulators per lane,
// held in AGPRs). K advances in stages of KT = 64 BPL elements (2 BPL MX
// blocks): FP4 lane slot g owns blocks g BPL .. g BPL + BPL - 1, and MFMA step
// kk (0 .. BPL-1) uses block g BPL + kk.
//
// One workgroup per CU walks a list of tiles. The stages of all its tiles form
// one stream: stage G of the stream lives in ring slot G mod NB, and the
// copies of stage G + NB - 1 (possibly of the next tile) are issued while
// stage G computes, so a tile starts with its first stages already in LDS.
//
// Global -> LDS moves use buffer loads that write LDS directly (no staging
// registers): each wave instruction fills 1 KiB of LDS, lane i writing bytes
// [16 i, 16 i + 16) of it, so the layout is set by choosing each lane's global
// address. Buffer resources carry the operand sizes: rows past M or N read as
// zero.
//
// Synchronisation, one barrier per stage: the barrier that opens stage G
// certifies that every wave's copies of stage G+1 have landed (each wave first
// waits for its own with s_waitcnt vmcnt) and that every wave has finished
// reading the slot about to be refilled (the one of stage G-1). Stage G then
// issues the copies of stage G+NB-1 between its first MFMAs, and while its
// MFMAs run it already reads the first fragments of stage G+1 from LDS, so the
// matrix pipe keeps working across the barrier.
//
// Epilogue: a tile's results leave during the next tile's first stage, whose
// first MFMA on each accumulator tile starts from zero: just before it the
// lane reads that accumulator tile out, and the values go through a small
// per-wave staging area to range-checked buffer stores (details at the
// stage loop below). The stores stay in flight while the next stages run:
// vmcnt counts loads and stores in issue order, so the wait of the stage
// after next allows the first stage's operations issued after its last copy
// to remain outstanding. Bias and per-token scales reach LDS by the same copy
// mechanism (issued one tile ahead), so the kernel issues no load whose wait
// the compiler would place.
//
// LDS rows hold one stage of one operand row (32, 64 or 128 bytes); their
// 16-byte chunks are XOR-permuted per row (swz) so that the 16 lanes of a
// ds_read_b128 phase reading one chunk of 16 consecutive rows hit 16 distinct
// bank groups.
//
// Tile order: workgroups are dealt round-robin to the 8 XCDs; XCD x owns a
// contiguous range of tiles in an order that walks groups of 4 tile-rows (m)
// per tile-column (n), and its workgroups take consecutive tiles of that
// range, so the 4 x 8 tiles in flight on one XCD share W and X panels in its
// L2 (groups of 4 measured 1-2.5% faster than 8 on random data, 16 and 32
// slower).

template <int MODE, int KT_, int NB_, int WAVES_>
struct PipeCfg {
  static constexpr int KT = KT_;                      // K elements per stage
  static constexpr int NB = NB_;                      // ring depth
  static constexpr int WAVES = WAVES_;                // waves per workgroup (one or two per SIMD)
  static constexpr int TM = WAVES == 8 ? 2 : 4;       // 32-row MFMA tiles of X per wave (W: always 4)
  static constexpr int NT = 4 * TM;                   // MFMAs per step and wave
  static constexpr int BPL = KT / 64;                 // blocks per lane slot per stage
  static constexpr int W_RB = KT / 2;                 // FP4 row bytes per stage
  static constexpr int X_RB = MODE == 0 ? KT / 2 : KT;  // FP4 / FP8 row bytes per stage
  static constexpr int W_OFF = 0;
  static constexpr int X_OFF = 256 * W_RB;
  static constexpr int WS_OFF = X_OFF + 256 * X_RB;   // 256 scale dwords (one group)
  static constexpr int XS_OFF = WS_OFF + 1024;
  static constexpr int STAGE = XS_OFF + (MODE == 0 ? 1024 : 0);
  static constexpr int W_INSTR = 256 * W_RB / 1024 / WAVES;   // 1 KiB copies per wave per stage
  static constexpr int X_INSTR = 256 * X_RB / 1024 / WAVES;
  static constexpr int S_INSTR = (MODE == 0 ? 8 : 4) / WAVES;  // 256 B scale copies per wave
  static constexpr int PER_WAVE = W_INSTR + X_INSTR + S_INSTR;
  static_assert(KT == 64 || KT == 128, "stage of one or two blocks per lane slot");
  static_assert(NB >= 3 && NB <= 8, "ring depth");
  static_assert(NB * STAGE <= 160 * 1024, "LDS");
  static_assert(KT == 128 || NB % 2 == 0, "half-group stages alternate scale bytes");
  static_assert(WAVES == 4 || (WAVES == 8 && MODE == 0), "two waves per SIMD: W4A4");
};

// LDS placement of 16-byte chunk c of `row` in a tile with rows of RB bytes:
// row-major, chunks XOR-permuted within the row by f(row). A ds_read_b128 of
// a fragment has 16 consecutive lanes reading the same chunk of 16 consecutive
// rows; f makes those 16 reads land in 16 different 16-byte bank groups of a
// 256-byte window (64 banks) and any 8 consecutive ones in 8 different groups
// of a 128-byte window (32 banks).
//   RB = 32  (2 chunks): bank group (2 row + c') mod 16 -> f = ((row>>2)^(row>>3)) & 1
//   RB = 64  (4 chunks): bank group (4 row + c') mod 16 -> f = ((row>>1)&3) ^ ((row>>3)&1)
//   RB = 128 (8 chunks): bank group (8 row + c') mod 16 -> f = ((row>>1)&7) ^ ((row&1)<<2)
template <int RB>
__device__ __forceinline__ int swz_f(int row) {
  if constexpr (RB == 128) return ((row >> 1) & 7) ^ ((row & 1) << 2);
  else if constexpr (RB == 64) return ((row >> 1) & 3) ^ ((row >> 3) & 1);
  else return ((row >> 2) ^ (row >> 3)) & 1;
}

template <int RB>
__device__ __forceinline__ int swz(int row, int c) {
  return row * RB + ((c ^ swz_f<RB>(row)) << 4);
}

// Inverse of swz: the (row, chunk) whose data belongs in 16-byte LDS slot `slot`.
template <int RB>
__device__ __forceinline__ void unswz(int slot, int& row, int& c) {
  constexpr int CPR = RB / 16;
  row = slot / CPR;
  c = (slot % CPR) ^ swz_f<RB>(row);
}

// Tile t of the grouped order: groups of 4 tile-rows, m fastest inside a group.
__device__ __forceinline__ void tile_of(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int G = 4;
  const int group = t / (G * tiles_n);
  const int first_m = group * G;
  const int gm = min(G, tiles_m - first_m);
  const int in = t - group * G * tiles_n;
  tm = first_m + in % gm;
  tn = in / gm;
}

#define MXQ_LDS __attribute__((address_space(3)))

constexpr int waitcnt_vm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// Buffer resource (V#) of a byte range: base, stride 0, size in bytes, and the
// gfx9 raw-buffer format word. Loads past `bytes` return zeros.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r.x = (int)(uint32_t)a;
  r.y = (int)(uint32_t)(a >> 32);
  r.z = (int)bytes;
  r.w = 0x00020000;
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)((const MXQ_LDS uint8_t*)p));
}

// One wave-wide copy from a buffer into LDS: lane i's 16 (or 4) bytes at byte
// offset `voff` of the resource land at LDS address lds + 16 i (4 i). The copy
// is written in asm so that the compiler's wait-count pass does not track it;
// the kernel orders it explicitly with s_waitcnt vmcnt + s_barrier. It has no
// register result, so nothing the compiler allocates can be overwritten while
// it is in flight; M0 needs one wait state before the copy reads it.
__device__ __forceinline__ void lds_dma16(const i32x4& rs, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds), "v"(voff), "s"(rs) : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const i32x4& rs, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :: "s"(lds), "v"(voff), "s"(rs) : "memory", "m0");
}

// Operand fragments of one MFMA step (4 W row groups, TM X row groups) and
// the scale registers of a stage (one 16-bit pair per row group for KT = 128,
// one byte for KT = 64).
template <int MODE, int TM>
struct StepData {
  uint4 a[4];
  uint4 b[MODE == 0 ? TM : 2 * TM];
};
template <int TM>
struct StageScales {
  uint32_t ws[4];
  uint32_t xs[TM];
};

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

// Static FP8 output (W4A8 GEMM writing the next W4A8 layer's activations):
// the division setup of the static quantizer, arranged for signed inputs. A
// zero scale maps every value to a signed zero (y = 0, hi = 0).
struct Fp8Out {
  float s, pre, ss, y, hi;
};

__device__ __forceinline__ Fp8Out fp8_out_setup(float amax) {
  const Fp8Row r = fp8_scale_setup(amax);
  Fp8Out o;
  o.s = r.s;
  o.pre = r.pre;
  o.ss = r.s == 0.0f ? 1.0f : r.ss;
  o.y = r.s == 0.0f ? 0.0f : r.y;
  o.hi = r.s == 0.0f ? 0.0f : r.hi;
  return o;
}

// Quotient x / s of a value that is exact in fp32 (a bf16 output), with the
// static quantizer's clamp at RN(448 ss) applied to both signs and x's sign
// put back afterwards (the correction step turns -0 into +0; for a nonzero
// quotient the sign is already x's). The magnitude equals that quantizer's
// quotient of |x|, so the E4M3FN codes are the same.
__device__ __forceinline__ float fp8_out_quotient(float x, const Fp8Out& o) {
  const float xs = __builtin_amdgcn_fmed3f(x * o.pre, -o.hi, o.hi);
  const float q0 = xs * o.y;
  const float rem = __builtin_fmaf(-q0, o.ss, xs);
  const float q = __builtin_fmaf(rem, o.y, q0);
  return as_float((as_uint(q) & 0x7FFFFFFFu) | (as_uint(x) & 0x80000000u));
}

// Two floats to packed bf16 (low half = a), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const v2f f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// Range-checked 16-byte store: offsets at or past the resource size are dropped.
// A store of more than 8 bytes reads its data registers one cycle late, so a
// VALU write to them right after it would change what is stored; the compiler
// guards that only for stores it knows about, so the wait state is part of the
// asm block.
// One accumulator register read into a VGPR at the point of use (left to the
// compiler, all 256 accumulators are copied out at once and spill).
__device__ __forceinline__ float acc_read(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

// Range-checked 4-byte store (one data register: no late read).
__device__ __forceinline__ void buf_store4(const i32x4& rs, uint32_t voff, uint32_t v) {
  asm volatile("buffer_store_dword %0, %1, %2, 0 offen" :: "v"(v), "v"(voff), "s"(rs) : "memory");
}

// Range-checked 8-byte store (no late read of its data registers).
__device__ __forceinline__ void buf_store8(const i32x4& rs, uint32_t voff, uint32_t lo, uint32_t hi) {
  const v2u d = {lo, hi};
  asm volatile("buffer_store_dwordx2 %0, %1, %2, 0 offen" :: "v"(d), "v"(voff), "s"(rs) : "memory");
}

__device__ __forceinline__ void buf_store16(const i32x4& rs, uint32_t voff, const uint4& v) {
  const i32x4 d = {(int)v.x, (int)v.y, (int)v.z, (int)v.w};
  asm volatile("buffer_store_dwordx4 %0, %1, %2, 0 offen\n\ts_nop 1" :: "v"(d), "v"(voff), "s"(rs) : "memory");
}

// QOUT: instead of y in bf16 the kernel writes the quantization of those bf16
// values in the activation format of a next layer of the same mode.
//   W4A4: MXFP4 codes in code panels of width 128 along N (y = codes, M N / 2
//         bytes) and group-major scales [N/128][M][4] (y_scales); N % 128 == 0.
//   W4A8: static FP8 with the scale out_amax / 448: codes [M][N] (y) and the
//         scale in every row of y_scales (float [M]).
// QOUT = 1 writes these; QOUT = 2 (W4A4, four waves) writes the MXFP4 codes
// of the transform_on activation instead: each row's 128 values of a code
// panel, as bf16, go through the unnormalized 128-point Walsh-Hadamard
// butterflies (h = 1, 2, 4, ..., 64 in that order, fp32, each a + b and
// a - b of the elements h apart), one fp32 multiply by the channel factor
// out_mult[n] (RN(t * mult + 0)) and rounding to bf16 before the MXFP4 rule,
// the arithmetic of the stand-alone transformed quantizer step for step.
//
// LRB (W4A4 only): SVDQuant's low-rank branch joins the sums. After a tile's
// K/128 code stages come r/32 more stages, one 32-wide rank panel each, with
// L2 [N][r] in the W role and T [M][r] in the X role: a 32-element bf16 panel
// row is 64 bytes, the size of a 128-element MXFP4 panel row, so the copies,
// the LDS layout and the fragment reads are those of a code stage, and only
// the MFMA changes (v_mfma_f32_32x32x16_bf16 into the same accumulators; its
// lane g supplies elements 8 g .. 8 g + 7 of a 16-element step, so the two
// steps of the stage read chunks {0, 2} and {1, 3} of the row, as both
// operands do). The stage's scale copies go out of range: they write zeros
// and read nothing, and keep the copy count of every stage the same.
template <int MODE, int KT, int NB, bool GELU, bool BIAS, int QOUT, bool LRB, int WAVES>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(WAVES / 4, WAVES / 4))) void
gemm_pipe_kernel(
    const uint8_t* __restrict__ wq, const uint8_t* __restrict__ ws,
    const uint8_t* __restrict__ aq, const void* __restrict__ asc,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, uint8_t* __restrict__ y_scales,
    const float* __restrict__ out_amax, int M, int N, int K, int tiles_m, int tiles_n,
    const uint16_t* __restrict__ lr_t, const uint16_t* __restrict__ lr_l2, int lr_rank,
    const float* __restrict__ out_mult) {
  using C = PipeCfg<MODE, KT, NB, WAVES>;
  constexpr int TM = C::TM, NT = C::NT;
  static_assert(!LRB || (MODE == 0 && KT == 128 && WAVES == 4), "the branch stages take the shape of a W4A4 code stage");
  static_assert(QOUT < 2 || (MODE == 0 && WAVES == 4 && !LRB), "transformed output: W4A4, four waves");
  // ring of NB stage slots, then two tile-parameter blocks: bias slice (512
  // bytes), a sink for the unused waves' copies (512), token scales (1024, FP8)
  // or channel factors (1024, transformed MXFP4 output)
  constexpr int P_BIAS = 0, P_SINK = 512, P_TOK = 1024, P_MULT = 1024;
  constexpr int PARAM_BYTES = MODE == 1 || QOUT == 2 ? 2048 : 1024;
  constexpr int PARAM_OFF = NB * C::STAGE;
  // The epilogue runs inside the next tile's first stage while the ring is
  // busy (see below), so it stages its results through a small area of its
  // own, per wave: W4A4 with four waves 32 rows x 144 bytes (a 64-column tile
  // pair); W4A8, and W4A4 with eight waves, 32 rows x 72 bytes (one 32-column
  // MFMA tile in bf16, or a tile pair of static FP8 codes: the larger W4A8
  // ring leaves 9 KiB, eight staging areas 18 KiB); MXFP4 output 32 rows x 80
  // bytes (one code panel of 32 rows).
  constexpr int EV_PITCH = MODE == 0 && WAVES == 4 ? 144 : 72;
  constexpr int EV_BYTES = 32 * (MODE == 0 && QOUT && EV_PITCH < 80 ? 80 : EV_PITCH);
  constexpr int EV_OFF = PARAM_OFF + 2 * PARAM_BYTES;
  static_assert(EV_OFF + WAVES * EV_BYTES <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[EV_OFF + WAVES * EV_BYTES];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int r = lane & 31;
  const int g = lane >> 5;
  const int wn = wave & 1;
  const int wm = wave >> 1;
  const int KB = K >> 5;
  const uint32_t w_row = (uint32_t)K >> 1;
  const uint32_t x_row = MODE == 0 ? ((uint32_t)K >> 1) : (uint32_t)K;
  const int nq = K / KT;                                   // code stages of a tile
  const int n_stages = nq + (LRB ? (lr_rank >> 5) : 0);   // + the branch's rank panels

  // This workgroup's tiles: first, first + stride, ... (count of them).
  const int total = tiles_m * tiles_n;
  const int P = gridDim.x;
  int first, stride, count;
  if ((P & 7) == 0 && total >= P) {
    const int x = blockIdx.x & 7, c = blockIdx.x >> 3, S = P >> 3;
    const int per = total >> 3, rem = total & 7;
    const int lo = x * per + min(x, rem), hi = (x + 1) * per + min(x + 1, rem);
    first = lo + c;
    stride = S;
    count = first < hi ? (hi - first + S - 1) / S : 0;
  } else {
    first = blockIdx.x;
    stride = P;
    count = (total - first + P - 1) / P;
  }
  first = __builtin_amdgcn_readfirstlane(first);
  count = __builtin_amdgcn_readfirstlane(count);

  // MXFP4 codes are K-panel-major with 128-element panels, one panel per
  // stage: stage s of a tile is the tile's 256 consecutive rows of panel s, one
  // contiguous 16 KiB block, so each wave-wide copy reads 1 KiB of consecutive
  // memory. FP8 activation codes are row-major, and a stage takes a full
  // 128-byte line of each row. Per-lane source offsets inside a tile's stage;
  // stage s adds s times the panel size (FP4) or the stage's row bytes (FP8).
  static_assert(KT == 128, "a stage is one 128-element code panel");
  uint32_t vw[C::W_INSTR], vx[C::X_INSTR];
#pragma unroll
  for (int q = 0; q < C::W_INSTR; ++q) {
    int row, c;
    unswz<C::W_RB>((wave * C::W_INSTR + q) * 64 + lane, row, c);
    vw[q] = (uint32_t)row * C::W_RB + (uint32_t)c * 16;
  }
#pragma unroll
  for (int q = 0; q < C::X_INSTR; ++q) {
    int row, c;
    unswz<C::X_RB>((wave * C::X_INSTR + q) * 64 + lane, row, c);
    vx[q] = (uint32_t)row * (MODE == 0 ? (uint32_t)C::X_RB : x_row) + (uint32_t)c * 16;
  }
  // branch stages: rank panel p of row `row` is at byte row * 2 r + 64 p
  const uint32_t lr_pitch = LRB ? (uint32_t)lr_rank * 2u : 0u;
  uint32_t vwl[LRB ? C::W_INSTR : 1], vxl[LRB ? C::X_INSTR : 1];
  if constexpr (LRB) {
#pragma unroll
    for (int q = 0; q < C::W_INSTR; ++q) vwl[q] = vw[q] / C::W_RB * lr_pitch + vw[q] % C::W_RB;
#pragma unroll
    for (int q = 0; q < C::X_INSTR; ++q) vxl[q] = vx[q] / C::X_RB * lr_pitch + vx[q] % C::X_RB;
  }
  const uint32_t w_panel = (uint32_t)N * C::W_RB;  // bytes of one code panel
  const uint32_t x_stage = MODE == 0 ? (uint32_t)M * C::X_RB : (uint32_t)C::X_RB;
  // Scales (group-major, 128-element groups): the tile's 256 dwords of group
  // gi are contiguous at byte (gi * rows + base) * 4; wave w copies dwords
  // 64 w .. 64 w + 63 of both operands (four waves), or of the W scales
  // (waves 0-3 of eight) or X scales (waves 4-7, dwords 64 (w - 4) ..). A
  // 64-element stage uses half of its group's bytes. Past the last row the
  // dwords belong to other rows (or read as zero at the end of the buffer) and
  // only feed outputs that are never stored.
  const uint32_t vs = (uint32_t)((wave & 3) * 64 + lane) * 4u;
  const uint32_t ws_group = (uint32_t)N * 4u;
  const uint32_t xs_group = (uint32_t)M * 4u;
  // eight waves: the operand whose scales this wave copies, fixed per wave
  // (chosen here with masks, so that the copy in the MFMA sequence is one
  // select on `live` like the others: a select of these inside the sequence
  // became a branch, which splits the interleaved block)
  const uint32_t sc_w = 0u - (uint32_t)(wave < 4);  // all ones: W scales
  const uint32_t sc_group = (ws_group & sc_w) | (xs_group & ~sc_w);
  const uint32_t sc_lds = (uint32_t)(wave < 4 ? C::WS_OFF : C::XS_OFF) + (uint32_t)(wave & 3) * 256u;

  // Whole-operand buffer resources: rows past M or N fall outside them.
  const i32x4 rw = make_rsrc(wq, w_row * (uint32_t)N);
  const i32x4 rx = make_rsrc(aq, x_row * (uint32_t)M);
  const i32x4 rws = make_rsrc(ws, (uint32_t)KB * (uint32_t)N);
  const i32x4 rxs = make_rsrc(asc, MODE == 0 ? (uint32_t)KB * (uint32_t)M : 0u);
  const i32x4 rl2 = make_rsrc(lr_l2, lr_pitch * (uint32_t)N);
  const i32x4 rlt = make_rsrc(lr_t, lr_pitch * (uint32_t)M);
  const i32x4 rsc = wave < 4 ? rws : rxs;  // eight waves: this wave's scale operand

  // ---- copy cursor: the stage (tile cp_k, stage cp_s) whose copies come
  // next, with the byte offsets of its tile in the W, X and scale operands.
  // The offsets of the tile after it are prepared off the MFMA path (in the
  // prologue and in each epilogue), so that moving on to the next tile takes
  // a few scalar selects and no branch: a branch between the MFMA steps
  // would split the block the reads and copies are interleaved in.
  const uint32_t lds_ring = lds_addr(ring);
  // first output column (nb) and row (mb) of tile k; zeros past the last tile
  auto tile_base = [&](int k, uint32_t& nb, uint32_t& mb) {
    int tm = 0, tn = 0;
    if (k < count) tile_of(first + k * stride, tiles_m, tiles_n, tm, tn);
    nb = (uint32_t)tn * 256u;
    mb = (uint32_t)tm * 256u;
  };
  int cp_k = 0, cp_s = 0;
  uint32_t cp_nb, cp_mb, nx_nb, nx_mb;  // the cursor's tile and the tile after it
  tile_base(0, cp_nb, cp_mb);
  tile_base(1, nx_nb, nx_mb);
  // Copy q (0 .. PER_WAVE-1) of the cursor's stage into ring slot `slot`.
  // Past the last tile the copies are still issued (so the wait counts stay
  // constant and the issue has no branch) but with 2^31 added to the offset,
  // beyond every resource's size (all below 2^31; the per-lane part is too,
  // so the sum does not wrap): the hardware then writes zeros to LDS without
  // reading memory. Offsets stay in the per-lane operand, the part the range
  // check covers; the scalar part is chosen with a scalar select.
  auto issue_one = [&](int q, int slot) {
    const bool live = cp_k < count;
    constexpr uint32_t oob = 0x80000000u;
    const uint32_t base = lds_ring + (uint32_t)slot * C::STAGE;
    // a branch stage (LRB): its rank panel, and its source rows 2 r bytes apart
    const bool br = LRB && cp_s >= nq;
    const uint32_t lr_off = LRB ? (uint32_t)(cp_s - nq) * 64u : 0u;
    if (q < C::W_INSTR) {
      const uint32_t so = live ? cp_nb * (uint32_t)C::W_RB + (uint32_t)cp_s * w_panel : oob;
      if constexpr (LRB) {
        const uint32_t sl = live ? cp_nb * lr_pitch + lr_off : oob;
        lds_dma16(br ? rl2 : rw, base + C::W_OFF + (wave * C::W_INSTR + q) * 1024, br ? vwl[q] + sl : vw[q] + so);
      } else {
        lds_dma16(rw, base + C::W_OFF + (wave * C::W_INSTR + q) * 1024, vw[q] + so);
      }
    } else if (q < C::W_INSTR + C::X_INSTR) {
      const int qx = q - C::W_INSTR;
      const uint32_t so =
          live ? cp_mb * (MODE == 0 ? (uint32_t)C::X_RB : x_row) + (uint32_t)cp_s * x_stage : oob;
      if constexpr (LRB) {
        const uint32_t sl = live ? cp_mb * lr_pitch + lr_off : oob;
        lds_dma16(br ? rlt : rx, base + C::X_OFF + (wave * C::X_INSTR + qx) * 1024, br ? vxl[qx] + sl : vx[qx] + so);
      } else {
        lds_dma16(rx, base + C::X_OFF + (wave * C::X_INSTR + qx) * 1024, vx[qx] + so);
      }
    } else if (WAVES == 8) {
      // the offset is below 2^31, so or-ing in the top bit puts it out of range
      // (a select of the computed offset here compiles to a branch)
      const uint32_t row0 = (cp_nb & sc_w) | (cp_mb & ~sc_w);
      const uint32_t so = (row0 * 4u + (uint32_t)cp_s * sc_group) | (live ? 0u : oob);
      lds_dma4(rsc, base + sc_lds, vs + so);
    } else if (q == C::W_INSTR + C::X_INSTR) {
      const uint32_t so = live && !br ? cp_nb * 4u + (uint32_t)(cp_s * KT / 128) * ws_group : oob;
      lds_dma4(rws, base + C::WS_OFF + wave * 256, vs + so);
    } else {
      const uint32_t so = live && !br ? cp_mb * 4u + (uint32_t)(cp_s * KT / 128) * xs_group : oob;
      lds_dma4(rxs, base + C::XS_OFF + wave * 256, vs + so);
    }
  };
  auto advance_cursor = [&] {
    const bool wrap = ++cp_s == n_stages;
    cp_s = wrap ? 0 : cp_s;
    cp_k += wrap ? 1 : 0;
    // a select on the values (written as a mask: the compiler turns the
    // conditional form into a select of addresses, which keeps them in memory)
    const uint32_t take = 0u - (uint32_t)wrap;
    cp_nb = (nx_nb & take) | (cp_nb & ~take);
    cp_mb = (nx_mb & take) | (cp_mb & ~take);
  };
  // Tile parameters of tile k into parameter block k & 1 (issued in stage 1
  // of tile k - 1, read in the first stage of tile k + 1): the bias slice
  // (waves 0, 1: 256 bytes each; the others copy nothing into the sink) and,
  // for FP8 activations, the 256 token scales, for the transformed MXFP4
  // output the 256 channel factors (256 bytes per wave). Always
  // EPI_PARAM_OPS copies per wave; no bias reads as zeros.
  constexpr int EPI_PARAM_OPS = MODE == 1 || QOUT == 2 ? 2 : 1;
  auto issue_params = [&](int k) {
    const bool live = k < count;
    int tm = 0, tn = 0;
    if (live) tile_of(first + k * stride, tiles_m, tiles_n, tm, tn);
    const uint32_t pb = lds_ring + PARAM_OFF + (uint32_t)(k & 1) * PARAM_BYTES;
    const uint32_t nb = (uint32_t)tn * 256u, mb = (uint32_t)tm * 256u;
    const i32x4 rb = make_rsrc(bias + nb, bias != nullptr ? ((uint32_t)N - nb) * 2u : 0u);
    lds_dma4(rb, pb + (wave < 2 ? P_BIAS + wave * 256 : P_SINK + ((wave - 2) & 1) * 256),
             live && wave < 2 ? (uint32_t)(wave * 256 + lane * 4) : 0x80000000u);
    if constexpr (MODE == 1) {
      const i32x4 rt = make_rsrc(static_cast<const uint8_t*>(asc) + mb * 4u, ((uint32_t)M - mb) * 4u);
      lds_dma4(rt, pb + P_TOK + wave * 256, live ? (uint32_t)(wave * 256 + lane * 4) : 0x80000000u);
    }
    if constexpr (QOUT == 2) {
      const i32x4 rm = make_rsrc(out_mult + nb, ((uint32_t)N - nb) * 4u);
      lds_dma4(rm, pb + P_MULT + wave * 256, live ? (uint32_t)(wave * 256 + lane * 4) : 0x80000000u);
    }
  };

  v16f acc[4][TM];

  const int wrow0 = wn * 128 + r;       // + 32 i
  const int xrow0 = wm * 32 * TM + r;   // + 32 j

  // LDS reads are issued one item at a time between MFMAs, in the order the
  // MFMAs consume them: an item is kind * 16 + index with kinds W fragment
  // (a[i]), X fragment (b[j]; for FP8 b[2j] / b[2j+1] are the two halves of
  // row group j), W scale (ws[i]) and X scale (xs[j]).
  constexpr int KA = 0, KBX = 16, KWS = 32, KXS = 48;
  // four waves: W4A4, W4A8; eight waves: W4A4 (two X row groups per wave)
  constexpr int OI = WAVES == 8 ? 2 : MODE;
  constexpr int DATA_ITEMS = OI == 0 ? 8 : OI == 1 ? 12 : 6;   // fragments of one step
  constexpr int STAGE_ITEMS = OI == 2 ? 12 : 16;               // step-0 fragments + scales of a stage
  constexpr int kStepOrder[3][12] = {
      {KA + 0, KBX + 0, KBX + 1, KBX + 2, KBX + 3, KA + 1, KA + 2, KA + 3, -1, -1, -1, -1},
      {KA + 0, KBX + 0, KBX + 1, KBX + 2, KBX + 3, KBX + 4, KBX + 5, KBX + 6, KBX + 7, KA + 1, KA + 2, KA + 3},
      {KA + 0, KBX + 0, KBX + 1, KA + 1, KA + 2, KA + 3, -1, -1, -1, -1, -1, -1}};
  constexpr int kStageOrder[3][16] = {
      {KA + 0, KBX + 0, KWS + 0, KXS + 0, KBX + 1, KXS + 1, KBX + 2, KXS + 2, KBX + 3, KXS + 3, KA + 1, KWS + 1,
       KA + 2, KWS + 2, KA + 3, KWS + 3},
      {KA + 0, KBX + 0, KBX + 1, KWS + 0, KBX + 2, KBX + 3, KBX + 4, KBX + 5, KBX + 6, KBX + 7, KA + 1, KWS + 1,
       KA + 2, KWS + 2, KA + 3, KWS + 3},
      {KA + 0, KBX + 0, KWS + 0, KXS + 0, KBX + 1, KXS + 1, KA + 1, KWS + 1, KA + 2, KWS + 2, KA + 3, KWS + 3,
       -1, -1, -1, -1}};
  // Copy q of a stage goes after MFMA slot floor(SPAN q / PER_WAVE). With
  // copies three or more stages ahead they spread over all 2 NT slots of the
  // stage (a burst would fill the vector memory queue and stall the wave that
  // also feeds the matrix pipe); two stages ahead, a copy issued late in its
  // stage would be waited for almost at once, so they go out first.
  constexpr int COPY_SPAN = NB - 1 >= 3 ? 2 * NT : C::PER_WAVE;
  constexpr auto kCopyAt = [] {
    std::array<int, 2 * NT> at{};
    for (int t = 0; t < 2 * NT; ++t) at[t] = -1;
    for (int q = 0; q < C::PER_WAVE; ++q) at[(COPY_SPAN * q) / C::PER_WAVE] = q;
    return at;
  }();
  static_assert(C::PER_WAVE <= 2 * NT, "one copy per MFMA slot at most");
  // Per-lane parts of the fragment offsets in a stage slot. Rows 32 apart
  // differ only in bits the chunk permutation does not use, so the offset of
  // row group idx is the lane part plus the constant 32 idx RB, which the
  // read instruction takes as its immediate offset.
  uint32_t lofs_a[C::BPL], lofs_b[C::BPL][MODE == 0 ? 1 : 2];
#pragma unroll
  for (int kk = 0; kk < C::BPL; ++kk) {
    lofs_a[kk] = C::W_OFF + swz<C::W_RB>(wrow0, g * C::BPL + kk);
    if constexpr (MODE == 0) {
      lofs_b[kk][0] = C::X_OFF + swz<C::X_RB>(xrow0, g * C::BPL + kk);
    } else {
      // FP8 slot h = g: half g of block kk (FP4 slot 0), then half g of block BPL+kk (slot 1)
      lofs_b[kk][0] = C::X_OFF + swz<C::X_RB>(xrow0, 2 * kk + g);
      lofs_b[kk][1] = C::X_OFF + swz<C::X_RB>(xrow0, 2 * (C::BPL + kk) + g);
    }
  }
  // scale dwords: row group idx adds 128 bytes; the lane's 16-bit pair is at + 2 g
  const uint32_t lofs_ws = C::WS_OFF + wrow0 * 4 + 2 * g, lofs_xs = C::XS_OFF + xrow0 * 4 + 2 * g;
  auto read_item = [&](const uint8_t* base, int kk, int half, int code, StepData<MODE, TM>& f,
                       StageScales<TM>& sc) {
    const int kind = code & ~15, idx = code & 15;
    if (kind == KA) {
      f.a[idx] = *reinterpret_cast<const uint4*>(base + lofs_a[kk] + 32 * idx * C::W_RB);
    } else if (kind == KBX) {
      if constexpr (MODE == 0)
        f.b[idx] = *reinterpret_cast<const uint4*>(base + lofs_b[kk][0] + 32 * idx * C::X_RB);
      else
        f.b[idx] = *reinterpret_cast<const uint4*>(base + lofs_b[kk][idx & 1] + 32 * (idx >> 1) * C::X_RB);
    } else {
      const bool is_w = kind == KWS;
      const uint32_t off = (is_w ? lofs_ws : lofs_xs) + 128 * idx;
      uint32_t v;
      if constexpr (KT == 128) v = *reinterpret_cast<const uint16_t*>(base + off);
      else v = base[off + 2 * half - g];
      if (is_w) sc.ws[idx] = v;
      else sc.xs[idx] = v;
    }
  };

  // The NT MFMAs of one step; after MFMA number k (0 .. NT-1) `between(k)`
  // may issue deferred operations, and the order is pinned by a scheduling
  // barrier so that the reads stay spread between the MFMAs.
  // `before(k)` runs before MFMA k; with `zero_tag` true the step starts the
  // tile's sums (accumulator input 0, an inline constant).
  // With `pin_tag` true each MFMA result passes through an empty asm
  // statement right after it: ordered with the other asm statements of the
  // step, the MFMA cannot be moved away from the work interleaved with it.
  // `order_tag` true takes the MFMAs j-outer (slot s = 4 j + i), so that a
  // 32-row group of the output is complete every 4 slots. Otherwise they run
  // i-outer, and in the steps that do not start the sums every other row runs
  // backwards (a snake): consecutive MFMAs then always share one operand, so
  // fewer operand bits switch (0.25-0.3% faster on the A14B shapes under the
  // power cap, measured interleaved; same sums). The first step keeps the
  // plain order, which the bf16 epilogues walk.
  auto mfma_step_x = [&](const StepData<MODE, TM>& f, const StageScales<TM>& sc, auto kk_tag, auto zero_tag,
                         auto pin_tag, auto order_tag, auto&& before, auto&& between) {
    constexpr int KK = decltype(kk_tag)::value;
    constexpr bool ZERO = decltype(zero_tag)::value;
    constexpr bool PIN = decltype(pin_tag)::value;
    constexpr bool JOUT = decltype(order_tag)::value;
    constexpr int SEL = KT == 128 ? KK : 0;
#pragma unroll
    for (int s = 0; s < NT; ++s) {
      const int i = JOUT ? (s & 3) : (s / TM);
      const int j = JOUT ? (s >> 2) : (!ZERO && (i & 1)) ? TM - 1 - s % TM : s % TM;
      {
        before(s);
        const v8i a = op_fp4(f.a[i]);
        if constexpr (MODE == 0)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, op_fp4(f.b[j]), ZERO ? v16f{} : acc[i][j],
                                                                      kFmtFp4, kFmtFp4, SEL, (int)sc.ws[i], SEL,
                                                                      (int)sc.xs[j]);
        else
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, op_fp8(f.b[2 * j], f.b[2 * j + 1]),
                                                                      ZERO ? v16f{} : acc[i][j], kFmtFp4, kFmtFp8,
                                                                      SEL, (int)sc.ws[i], SEL, (int)kUnitScales);
        if constexpr (PIN && WAVES == 4) asm volatile("" ::"a"(acc[i][j]));
        // (one element suffices to keep the MFMA in place; a whole 16-float
        // vector is no valid operand of the host's "v" constraint)
        if constexpr (PIN && WAVES == 8) asm volatile("" ::"v"(acc[i][j][0]));
        between(s);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  auto mfma_step = [&](const StepData<MODE, TM>& f, const StageScales<TM>& sc, auto kk_tag, auto&& between) {
    mfma_step_x(f, sc, kk_tag, std::false_type{}, std::false_type{}, std::false_type{}, [](int) {}, between);
  };
  // the 16 MFMAs of one step of a branch stage: bf16 operands, no scales
  auto mfma_step_bf = [&](const StepData<MODE, TM>& f, auto&& between) {
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const int i = s >> 2, j = s & 3;
      if constexpr (MODE == 0)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f.a[i]),
                                                            __builtin_bit_cast(bf16x8, f.b[j]), acc[i][j], 0, 0, 0);
      between(s);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Epilogue stores per wave and tile (W4A4: 32 bf16 stores with four waves,
  // 2 per MFMA tile with eight, or with QOUT per 32-row group two 1 KiB code
  // stores and one scale store; W4A8: 32 bf16 stores, or with QOUT 2 per tile
  // pair and one store of row scales), the same whatever the shape: rows past
  // M and columns past N get an offset the range check drops.
  constexpr int EPI_STORES = MODE == 0 ? (QOUT ? 3 * TM : WAVES == 4 ? 32 : 2 * NT) : (QOUT ? 17 : 32);
  constexpr int EPI_OPS = EPI_STORES + EPI_PARAM_OPS;
  // Output resource of one tile's rows for the row-major outputs (bf16, or
  // static FP8 codes): its base is the tile's first row, so the offsets stay
  // far below 2^31 for outputs of any size, and rows past M fall past its end
  // (dropped by the range check).
  constexpr uint32_t Y_ELT = MODE == 1 && QOUT ? 1u : 2u;
  auto tile_out = [&](int ptm) {
    const int rows = min(256, M - ptm * 256);
    return make_rsrc(reinterpret_cast<const uint8_t*>(y) + (size_t)ptm * 256u * (size_t)N * Y_ELT,
                     (uint32_t)rows * (uint32_t)N * Y_ELT);
  };
  Fp8Out fo{};
  if constexpr (MODE == 1 && QOUT) fo = fp8_out_setup(*out_amax);

  constexpr int D = NB - 1;  // copies run D stages ahead of the stage computed
  constexpr int WAIT_BASE = (D - 2) * C::PER_WAVE;
  static_assert(WAIT_BASE + EPI_OPS <= 63, "vmcnt range");

  // prologue: tile parameters of the first tile, copies of stages 0 .. D-1;
  // stages 0 and 1 must have landed before the first fragments are read
  issue_params(0);
#pragma unroll
  for (int st = 0; st < D; ++st) {
#pragma unroll
    for (int q = 0; q < C::PER_WAVE; ++q) issue_one(q, st);
    advance_cursor();
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(WAIT_BASE));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  StepData<MODE, TM> cur;
  StageScales<TM> cur_sc;
#pragma unroll
  for (int k = 0; k < STAGE_ITEMS; ++k) read_item(ring, 0, 0, kStageOrder[OI][k], cur, cur_sc);

  {
    // ---- The epilogue of tile t-1 runs inside the first stage of
    // tile t. Before MFMA (i, j) of that stage's first step (which starts the
    // new sums from zero) the lane reads accumulator tile (i, j) of tile t-1
    // out of its registers, adds the bias, applies GELU and packs bf16 pairs;
    // v_permlane32_swap then gives each lane 16 contiguous bytes of one row
    // (columns 16 u + 8 g .. + 7 of the 32-column tile). When both tiles of a
    // column pair (i = 2h, 2h+1) of row group j are ready they go through the
    // wave's staging area (32 rows x 64 columns) and leave as 4 stores of 8
    // rows x 128 contiguous bytes, one MFMA slot later. The matrix pipe keeps
    // working while the vector unit does this. Tile 0's first stage has no
    // previous tile (its stores are dropped), and one extra stage after the
    // last tile, computing on zeros, carries the last tile's epilogue.
    // W4A8 (bf16 output) does the same per MFMA tile: the per-token scale of
    // the lane's row, bias and GELU, then the tile's 32 rows x 64 bytes go
    // through the staging area and leave as 2 stores of 16 rows x 64 bytes
    // one MFMA slot later.
    uint8_t* ev_region = ring + EV_OFF + wave * EV_BYTES;
    // bias of the lane's 16 columns of MFMA tile row group i, in accumulator
    // order (q = 4 t + c: column 32 i + 8 t + 4 g + c)
    auto ev_bias = [&](const uint8_t* prm, int i, v16f& b) {
#pragma unroll
      for (int t2 = 0; t2 < 4; ++t2) {
        const uint2 bb = *reinterpret_cast<const uint2*>(prm + P_BIAS + (wn * 128 + 32 * i + 8 * t2 + 4 * g) * 2);
        b[4 * t2 + 0] = as_float(bb.x << 16);
        b[4 * t2 + 1] = as_float(bb.x & 0xFFFF0000u);
        b[4 * t2 + 2] = as_float(bb.y << 16);
        b[4 * t2 + 3] = as_float(bb.y & 0xFFFF0000u);
      }
    };
    // accumulator tile (i, j) of the finished tile (x the row's token scale
    // for W4A8, + bias) -> 8 bf16 pairs: pair h of run t holds columns
    // 8 t + 4 g + 2 h, + 1
    auto ev_tile = [&](int i, int j, const v16f& b, float sm, uint32_t (&pk)[4][2]) {
#pragma unroll
      for (int t2 = 0; t2 < 4; ++t2)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          // four waves hold the sums in accumulator registers, eight in VGPRs
          float v0, v1;
          if constexpr (WAVES == 4) {
            v0 = acc_read(acc[i][j][4 * t2 + 2 * h]);
            v1 = acc_read(acc[i][j][4 * t2 + 2 * h + 1]);
          } else {
            v0 = acc[i][j][4 * t2 + 2 * h];
            v1 = acc[i][j][4 * t2 + 2 * h + 1];
          }
          if constexpr (MODE == 1) {
            v0 = BIAS ? __builtin_fmaf(v0, sm, b[4 * t2 + 2 * h]) : v0 * sm;
            v1 = BIAS ? __builtin_fmaf(v1, sm, b[4 * t2 + 2 * h + 1]) : v1 * sm;
          } else if constexpr (BIAS) {
            v0 += b[4 * t2 + 2 * h];
            v1 += b[4 * t2 + 2 * h + 1];
          }
          if constexpr (GELU) {
            v0 = gelu_tanh_dev(v0);
            v1 = gelu_tanh_dev(v1);
          }
          pk[t2][h] = pack_bf16x2(v0, v1);
        }
    };
    // staging area: row r holds the 64 columns of tiles 2h, 2h+1; the lane's
    // run t of tile ii is 8 bytes at column 32 ii + 8 t + 4 g
    auto ev_unit_write = [&](const uint32_t (&p0)[4][2], const uint32_t (&p1)[4][2]) {
#pragma unroll
      for (int t2 = 0; t2 < 4; ++t2) {
        *reinterpret_cast<uint2*>(ev_region + r * EV_PITCH + 16 * t2 + 8 * g) = make_uint2(p0[t2][0], p0[t2][1]);
        *reinterpret_cast<uint2*>(ev_region + r * EV_PITCH + 64 + 16 * t2 + 8 * g) = make_uint2(p1[t2][0], p1[t2][1]);
      }
    };
    auto ev_unit_read = [&](uint4 (&rd)[4]) {
#pragma unroll
      for (int it = 0; it < 4; ++it)
        rd[it] = *reinterpret_cast<const uint4*>(ev_region + (8 * it + (lane >> 3)) * EV_PITCH + (lane & 7) * 16);
    };
    // W4A8: one tile's 32 rows x 64 bytes; lane l reads 16 bytes of row
    // 16 st + l / 4 at byte 16 (l % 4), as two 8-byte reads (the 72-byte
    // pitch keeps 8-byte alignment and spreads the rows over the banks)
    auto ev8_write = [&](const uint32_t (&p)[4][2]) {
#pragma unroll
      for (int t2 = 0; t2 < 4; ++t2)
        *reinterpret_cast<uint2*>(ev_region + r * EV_PITCH + 16 * t2 + 8 * g) = make_uint2(p[t2][0], p[t2][1]);
    };
    auto ev8_read = [&](uint4 (&rd)[2]) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const uint8_t* src = ev_region + (16 * st + (lane >> 2)) * EV_PITCH + (lane & 3) * 16;
        const uint2 lo = *reinterpret_cast<const uint2*>(src);
        const uint2 hi = *reinterpret_cast<const uint2*>(src + 8);
        rd[st] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
    };

    // The next tile's parameters are copied at the start of stage 1 (below),
    // so the first stage issues copies and stores only.
    constexpr int D_SLACK1 = EPI_STORES;  // a wait that every op of the first stage may outlast
    // The stage after the next may leave outstanding the ops of the first
    // stage issued after its last copy, and those of stage 1 (its parameter
    // copies come before its stage copies): W4A4 issues every epilogue store
    // before its last copy (slot > 16), W4A8 issues its 13 copies in slots
    // 0..12 and the stores of tile t (2 each) after slot t + 1, tile 15's in
    // the second step, so tiles 11..15 come after the last copy.
    constexpr int kLastCopySlot = COPY_SPAN * (C::PER_WAVE - 1) / C::PER_WAVE;
    static_assert(MODE == 1 || kLastCopySlot > NT, "W4A4 epilogue stores end in slot NT");
    static_assert(MODE == 0 || (kLastCopySlot >= 1 && kLastCopySlot <= 16), "W4A8 copies within the first step");
    // (W4A8 static FP8 output: tile pairs complete at slots 4 + j and 12 + j
    // and are stored one slot later, so 4 pairs after slot 12.)
    constexpr int D_SLACK2 = MODE == 0 ? EPI_PARAM_OPS  // stage 1 (D = 3): parameters + a stage of copies
                             : QOUT    ? 2 * 4          // D = 2: stage 0's late stores only
                                       : 2 * (17 - kLastCopySlot);
    static_assert(MODE == 0 || !QOUT || kLastCopySlot == 12, "W4A8 static-FP8 store schedule");

    int slot = 0;  // ring slot of the stage being computed
    auto run_stage = [&](int tile_k, int s_in, auto first_tag, auto br_tag) {
      constexpr bool FIRST = decltype(first_tag)::value;
      constexpr bool BR = decltype(br_tag)::value;
      if (tile_k > 0 || s_in > 0) {
        // the stage after the first one may leave all of the first stage's
        // operations outstanding; the one after that, those issued after its
        // last copy
        if (s_in >= 1 && s_in <= D - 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(WAIT_BASE + D_SLACK1));
        else if (s_in == D - 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(WAIT_BASE + D_SLACK2));
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm(WAIT_BASE));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      }
      // The parameters of tile k + 1 go into the block that the epilogue of
      // tile k - 1 read during the first stage; the barrier that opens stage 1
      // is the first point at which every wave has finished those reads (the
      // block is next read in the first stage of tile k + 2).
      if constexpr (!FIRST) {
        if (s_in == 1) issue_params(tile_k + 1);
      }
      const int G = tile_k * n_stages + s_in;
      const int slot_next = slot + 1 == NB ? 0 : slot + 1;
      const int slot_refill = slot == 0 ? NB - 1 : slot - 1;  // (G + D) mod NB
      const uint8_t* here = ring + slot * C::STAGE;
      const uint8_t* next = ring + slot_next * C::STAGE;
      const int next_half = (G + 1) & 1;
      StepData<MODE, TM> nxt;
      StageScales<TM> nxt_sc;
      auto between0 = [&](int k) {
        if (k < DATA_ITEMS) read_item(here, 1, 0, kStepOrder[OI][k], nxt, nxt_sc);
        if (kCopyAt[k] >= 0) issue_one(kCopyAt[k], slot_refill);
      };
      // the next stage's STAGE_ITEMS reads spread over the NT slots of step 1
      auto between1 = [&](int k) {
#pragma unroll
        for (int it = k * STAGE_ITEMS / NT; it < (k + 1) * STAGE_ITEMS / NT; ++it)
          read_item(next, 0, next_half, kStageOrder[OI][it], cur, cur_sc);
        if (kCopyAt[NT + k] >= 0) issue_one(kCopyAt[NT + k], slot_refill);
      };
      if constexpr (!FIRST && BR) {
        mfma_step_bf(cur, between0);
        mfma_step_bf(nxt, between1);
      } else if constexpr (!FIRST) {
        mfma_step(cur, cur_sc, std::integral_constant<int, 0>{}, between0);
        const StageScales<TM> sc1 = cur_sc;
        mfma_step(nxt, sc1, std::integral_constant<int, 1>{}, between1);
      } else {
        // the cursor is in this tile (stage D): the tile it moves to next is
        // tile_k + 1
        tile_base(cp_k + 1, nx_nb, nx_mb);
        const bool ev_live = tile_k > 0;
        int ptm = 0, ptn = 0;
        if (ev_live) tile_of(first + (tile_k - 1) * stride, tiles_m, tiles_n, ptm, ptn);
        if constexpr (MODE == 0 && QOUT) {
          // MXFP4 output. The wave's 128 columns are one code panel of the
          // output (64 bytes per row, rows contiguous) and one scale dword per
          // row. The first step runs j-outer: before MFMA (i, j) the lane turns
          // accumulator tile (i, j) into bf16 pairs (bias, GELU) exactly as
          // the bf16 epilogue would, takes the block amax over its 16 values and
          // its partner lane's 16 (lane +- 32: together the 32 columns of the
          // tile's row), and converts them with the quantizer's scaled
          // conversion. A lane swap and two byte permutes leave each lane 8
          // contiguous code bytes of its row; they go into the staging area
          // (32 rows x 64 bytes), and after the 4 tiles of row group j the
          // group's 2 KiB leave as two 1 KiB stores, with the 32 scale dwords,
          // one slot later.
          constexpr int QP = 80;  // staging pitch: 64 bytes + 16 (16-byte aligned rows)
          const int n_q = ptn * 256 + wn * 128;
          const uint32_t q_bad = ev_live && n_q < N ? 0u : 0x80000000u;
          const uint32_t q_pan = (uint32_t)(n_q >> 7);
          const int m_q = ptm * 256 + wm * 32 * TM;
          const i32x4 rq = make_rsrc(y, (uint32_t)M * (uint32_t)N / 2u);
          const i32x4 rsq = make_rsrc(y_scales, (uint32_t)(N >> 7) * (uint32_t)M * 4u);
          const uint8_t* prm = ring + PARAM_OFF + ((tile_k - 1) & 1) * PARAM_BYTES;
          // bias of the four column tiles: held for the stage with four waves,
          // read per tile with eight (whose 256 registers have no room for them)
          // and with the transform (whose 64 rotated values take that room)
          constexpr bool BQ4 = WAVES == 4 && QOUT == 1;
          v16f bq[BQ4 ? 4 : 1];
          if constexpr (BIAS && BQ4) {
#pragma unroll
            for (int i = 0; i < 4; ++i) ev_bias(prm, i, bq[i]);
          }
          uint4 rd[2];
          uint32_t sbs = 0, sbs_done = 0;
          auto group_store = [&](int j) {
#pragma unroll
            for (int it = 0; it < 2; ++it) {
              const int row = m_q + 32 * j + 16 * it + (lane >> 2);
              const uint32_t off = q_pan * 64u * (uint32_t)M + (uint32_t)row * 64u + (uint32_t)(lane & 3) * 16u;
              buf_store16(rq, row < M ? (off | q_bad) : 0x80000000u, rd[it]);
            }
            const int srow = m_q + 32 * j + r;
            const uint32_t soff = (q_pan * (uint32_t)M + (uint32_t)srow) * 4u;
            buf_store4(rsq, g == 0 && srow < M ? (soff | q_bad) : 0x80000000u, sbs_done);
          };
          // E8M0 scale byte of a 32-column block from the lane's 8 bf16 pairs
          // and its partner's (lane +- 32)
          auto block_scale = [&](const uint32_t (&pk)[4][2]) {
            typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
            u16x2 m2 = {0, 0};
#pragma unroll
            for (int t2 = 0; t2 < 4; ++t2)
#pragma unroll
              for (int h = 0; h < 2; ++h)
                m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, pk[t2][h] & 0x7FFF7FFFu));
            uint32_t am = umax((uint32_t)m2.x, (uint32_t)m2.y);
            const auto sw = __builtin_amdgcn_permlane32_swap(am, am, false, false);
            am = umax(am, g ? (uint32_t)sw[0] : (uint32_t)sw[1]);
            return mx_scale_byte(am);
          };
          // Transformed output: tile i's values of the lane's row after the
          // butterflies h = 1 .. 16 (and later 32, 64), hv[i][4 t + c]:
          // c = 0, 1 column 32 i + 8 t + 2 g + c, c = 2, 3 column
          // 32 i + 8 t + 4 + 2 g + c - 2 of the code panel.
          float hv[4][16];
          auto bfly = [](float& a, float& b) {
            const float x0 = a, x1 = b;
            a = x0 + x1;
            b = x0 - x1;
          };
          // tile ii of the row group: factors, bf16, MXFP4 codes into staging.
          // (These two must be inlined: their tile index has to be a constant
          // where it indexes the accumulators and hv, or both go to memory.)
          auto quant_rotated = [&](int ii) __attribute__((always_inline)) {
            uint32_t pk[4][2];  // [t][0]: columns 8 t + 2 g, + 1; [t][1]: + 4
#pragma unroll
            for (int t2 = 0; t2 < 4; ++t2)
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                const float2 m = *reinterpret_cast<const float2*>(
                    prm + P_MULT + (wn * 128 + 32 * ii + 8 * t2 + 4 * h + 2 * g) * 4);
                // RN(t * mult + 0): an exact zero becomes +0, as in the
                // stand-alone quantizer
                pk[t2][h] = pack_bf16x2(__builtin_fmaf(hv[ii][4 * t2 + 2 * h], m.x, 0.0f),
                                        __builtin_fmaf(hv[ii][4 * t2 + 2 * h + 1], m.y, 0.0f));
              }
            const uint32_t sb = block_scale(pk);
            const float scq = as_float(sb << 23);
            // byte 4 t + 2 h + g of the row's 16 code bytes per pair: code
            // dword e0 holds runs t = 0, 1, e1 runs 2, 3 (bytes of one parity)
            uint32_t e0 = 0, e1 = 0;
            e0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(e0, __builtin_bit_cast(bf16x2, pk[0][0]), scq, 0);
            e0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(e0, __builtin_bit_cast(bf16x2, pk[0][1]), scq, 1);
            e0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(e0, __builtin_bit_cast(bf16x2, pk[1][0]), scq, 2);
            e0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(e0, __builtin_bit_cast(bf16x2, pk[1][1]), scq, 3);
            e1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(e1, __builtin_bit_cast(bf16x2, pk[2][0]), scq, 0);
            e1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(e1, __builtin_bit_cast(bf16x2, pk[2][1]), scq, 1);
            e1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(e1, __builtin_bit_cast(bf16x2, pk[3][0]), scq, 2);
            e1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(e1, __builtin_bit_cast(bf16x2, pk[3][1]), scq, 3);
            // after the swap the lower lane holds the even and odd bytes 0 .. 7,
            // the upper lane bytes 8 .. 15; interleaving them gives each lane 8
            // contiguous bytes
            const auto pq = __builtin_amdgcn_permlane32_swap(e0, e1, false, false);
            const uint32_t wlo = __builtin_amdgcn_perm((uint32_t)pq[1], (uint32_t)pq[0], 0x05010400u);
            const uint32_t whi = __builtin_amdgcn_perm((uint32_t)pq[1], (uint32_t)pq[0], 0x07030602u);
            *reinterpret_cast<uint2*>(ev_region + r * QP + 16 * ii + 8 * g) = make_uint2(wlo, whi);
            sbs |= sb << (8 * ii);
          };
          auto beforeh = [&](int sl) __attribute__((always_inline)) {
            const int i = sl & 3, j = sl >> 2;
            // accumulator tile (i, j) -> bias, GELU, bf16 (as ev_tile, with the
            // bias read per run of 4 columns: the rotated values leave no room
            // for a whole tile's)
            uint32_t pk[4][2];
#pragma unroll
            for (int t2 = 0; t2 < 4; ++t2) {
              uint2 bb = make_uint2(0u, 0u);
              if constexpr (BIAS)
                bb = *reinterpret_cast<const uint2*>(prm + P_BIAS + (wn * 128 + 32 * i + 8 * t2 + 4 * g) * 2);
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                float v0 = acc_read(acc[i][j][4 * t2 + 2 * h]);
                float v1 = acc_read(acc[i][j][4 * t2 + 2 * h + 1]);
                if constexpr (BIAS) {
                  const uint32_t b2 = h ? bb.y : bb.x;
                  v0 += as_float(b2 << 16);
                  v1 += as_float(b2 & 0xFFFF0000u);
                }
                if constexpr (GELU) {
                  v0 = gelu_tanh_dev(v0);
                  v1 = gelu_tanh_dev(v1);
                }
                pk[t2][h] = pack_bf16x2(v0, v1);
              }
            }
            // the bf16 values of columns 8 t + 4 g + c, exactly, in fp32
            float f[4][4];
#pragma unroll
            for (int t2 = 0; t2 < 4; ++t2) {
              f[t2][0] = as_float(pk[t2][0] << 16);
              f[t2][1] = as_float(pk[t2][0] & 0xFFFF0000u);
              f[t2][2] = as_float(pk[t2][1] << 16);
              f[t2][3] = as_float(pk[t2][1] & 0xFFFF0000u);
              bfly(f[t2][0], f[t2][1]);  // h = 1
              bfly(f[t2][2], f[t2][3]);
              bfly(f[t2][0], f[t2][2]);  // h = 2
              bfly(f[t2][1], f[t2][3]);
            }
            // h = 4 pairs the lane with its partner: one swap of columns c and
            // c + 2 gives the lower lane both halves' column c and the upper
            // lane both halves' column c + 2, the g = 0 element first
#pragma unroll
            for (int t2 = 0; t2 < 4; ++t2)
#pragma unroll
              for (int c = 0; c < 2; ++c) {
                const auto sw = __builtin_amdgcn_permlane32_swap(as_uint(f[t2][c]), as_uint(f[t2][c + 2]), false, false);
                const float lo = as_float((uint32_t)sw[0]), hi = as_float((uint32_t)sw[1]);
                hv[i][4 * t2 + c] = lo + hi;
                hv[i][4 * t2 + 2 + c] = lo - hi;
              }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              bfly(hv[i][e], hv[i][4 + e]);  // h = 8
              bfly(hv[i][8 + e], hv[i][12 + e]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              bfly(hv[i][e], hv[i][8 + e]);  // h = 16
              bfly(hv[i][4 + e], hv[i][12 + e]);
            }
            if (i & 1) {
#pragma unroll
              for (int e = 0; e < 16; ++e) bfly(hv[i - 1][e], hv[i][e]);  // h = 32
            }
            if (i == 3) {
#pragma unroll
              for (int e = 0; e < 16; ++e) {
                bfly(hv[0][e], hv[2][e]);  // h = 64
                bfly(hv[1][e], hv[3][e]);
              }
#pragma unroll
              for (int ii = 0; ii < 4; ++ii) quant_rotated(ii);
            }
          };
          auto beforeq = [&](int sl) {
            const int i = sl & 3, j = sl >> 2;
            uint32_t pk[4][2];
            if constexpr (WAVES == 4) {
              ev_tile(i, j, bq[i], 1.0f, pk);
            } else {
              if constexpr (BIAS) ev_bias(prm, i, bq[0]);
              ev_tile(i, j, bq[0], 1.0f, pk);
            }
            const uint32_t sb = block_scale(pk);
            const float scq = as_float(sb << 23);
            uint32_t e0 = 0, e1 = 0;
            e0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(e0, __builtin_bit_cast(bf16x2, pk[0][0]), scq, 0);
            e0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(e0, __builtin_bit_cast(bf16x2, pk[0][1]), scq, 1);
            e0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(e0, __builtin_bit_cast(bf16x2, pk[1][0]), scq, 2);
            e0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(e0, __builtin_bit_cast(bf16x2, pk[1][1]), scq, 3);
            e1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(e1, __builtin_bit_cast(bf16x2, pk[2][0]), scq, 0);
            e1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(e1, __builtin_bit_cast(bf16x2, pk[2][1]), scq, 1);
            e1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(e1, __builtin_bit_cast(bf16x2, pk[3][0]), scq, 2);
            e1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(e1, __builtin_bit_cast(bf16x2, pk[3][1]), scq, 3);
            // lane g = 0 holds code bytes 4t + {0, 1} (t = 0..3) of the row's 16
            // bytes of tile i, lane g = 1 bytes 4t + {2, 3}: after the swap the
            // lower lane has both halves' t = 0, 1 bytes, the upper lane t = 2, 3
            const auto pq = __builtin_amdgcn_permlane32_swap(e0, e1, false, false);
            const uint32_t wlo = __builtin_amdgcn_perm((uint32_t)pq[1], (uint32_t)pq[0], 0x05040100u);
            const uint32_t whi = __builtin_amdgcn_perm((uint32_t)pq[1], (uint32_t)pq[0], 0x07060302u);
            *reinterpret_cast<uint2*>(ev_region + r * QP + 16 * i + 8 * g) = make_uint2(wlo, whi);
            sbs |= sb << (8 * i);
          };
          auto afterq = [&](int sl) {
            between0(sl);
            if (sl >= 4 && (sl & 3) == 0) group_store((sl >> 2) - 1);
            if ((sl & 3) == 3) {
              __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
              for (int it = 0; it < 2; ++it)
                rd[it] = *reinterpret_cast<const uint4*>(ev_region + (16 * it + (lane >> 2)) * QP + (lane & 3) * 16);
              // the next group's writes stay behind these reads
              __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
              sbs_done = sbs;
              sbs = 0;
            }
          };
          mfma_step_x(cur, cur_sc, std::integral_constant<int, 0>{}, std::true_type{}, std::true_type{},
                      std::true_type{}, [&](int sl) {
                        if constexpr (QOUT == 2) beforeh(sl);
                        else beforeq(sl);
                      }, afterq);
          const StageScales<TM> sc1 = cur_sc;
          mfma_step_x(nxt, sc1, std::integral_constant<int, 1>{}, std::false_type{}, std::true_type{},
                      std::false_type{}, [](int) {}, [&](int k) {
                        between1(k);
                        if (k == 0) group_store(TM - 1);
                      });
        } else if constexpr (MODE == 1 && QOUT) {
          // W4A8 with static FP8 output: each tile's bf16 values (token scale,
          // bias, GELU) become the static quantizer's codes, 4 bytes per run of
          // 4 columns. Tile (2h, j)'s codes wait in registers for tile
          // (2h + 1, j) (4 slots later, i outer); the pair's 32 rows x 64
          // bytes go through the staging area and leave as two stores of 16
          // rows x 64 bytes one slot later. The row scales (out_amax / 448)
          // leave in one store per wave, from the tiles of the first column.
          const i32x4 ry = tile_out(ptm);
          const int ev_m0 = wm * 128 + (lane >> 2);  // row in the tile, + 32 j + 16 st
          const int ev_n0 = ptn * 256 + wn * 128 + (lane & 3) * 16;  // + 64 h
          const uint8_t* prm = ring + PARAM_OFF + ((tile_k - 1) & 1) * PARAM_BYTES;
          float sm[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) sm[j] = *reinterpret_cast<const float*>(prm + P_TOK + (wm * 128 + 32 * j + r) * 4);
          v16f c_cur, c_nxt;
          if constexpr (BIAS) ev_bias(prm, 0, c_cur);
          uint32_t q_even[4][4];  // codes of tile (2h, j), per j, per run
          uint32_t q_cur[4];
          uint4 rd[2];
          auto pair_store = [&](int h, int j) {
            const uint32_t bad = ev_live && ev_n0 + 64 * h < N ? 0u : 0x80000000u;
#pragma unroll
            for (int st = 0; st < 2; ++st) {
              const uint32_t off = (uint32_t)(ev_m0 + 32 * j + 16 * st) * (uint32_t)N + (uint32_t)(ev_n0 + 64 * h);
              buf_store16(ry, off | bad, rd[st]);
            }
          };
          auto before8 = [&](int k) {
            const int i = k >> 2, j = k & 3;
            if (BIAS && j == 0 && i > 0) c_cur = c_nxt;
            uint32_t pk[4][2];
            ev_tile(i, j, c_cur, sm[j], pk);
#pragma unroll
            for (int t2 = 0; t2 < 4; ++t2) {
              const float q0 = fp8_out_quotient(as_float(pk[t2][0] << 16), fo);
              const float q1 = fp8_out_quotient(as_float(pk[t2][0] & 0xFFFF0000u), fo);
              const float q2 = fp8_out_quotient(as_float(pk[t2][1] << 16), fo);
              const float q3 = fp8_out_quotient(as_float(pk[t2][1] & 0xFFFF0000u), fo);
              uint32_t o = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
              q_cur[t2] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, (int)o, true);
            }
          };
          auto after8 = [&](int k) {
            const int i = k >> 2, j = k & 3;
            between0(k);
            if (k == 0) {
              const int m = ptm * 256 + t;
              const i32x4 rs = make_rsrc(y_scales, (uint32_t)M * 4u);
              buf_store4(rs, ev_live && ptn == 0 && m < M ? (uint32_t)m * 4u : 0x80000000u, as_uint(fo.s));
            }
            // the pair completed in the previous slot
            if (k >= 5 && k <= 8) pair_store(0, k - 5);
            if (k >= 13) pair_store(1, k - 13);
            if ((i & 1) == 0) {
#pragma unroll
              for (int t2 = 0; t2 < 4; ++t2) q_even[j][t2] = q_cur[t2];
            } else {
              // staging row r: bytes 8 t + 4 g of tile 2h, 32 + 8 t + 4 g of tile 2h + 1
#pragma unroll
              for (int t2 = 0; t2 < 4; ++t2) {
                *reinterpret_cast<uint32_t*>(ev_region + r * EV_PITCH + 8 * t2 + 4 * g) = q_even[j][t2];
                *reinterpret_cast<uint32_t*>(ev_region + r * EV_PITCH + 32 + 8 * t2 + 4 * g) = q_cur[t2];
              }
              __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
              ev8_read(rd);
              // the next pair's writes stay behind these reads
              __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            }
            if (BIAS && j == 1 && i < 3) ev_bias(prm, i + 1, c_nxt);
          };
          mfma_step_x(cur, cur_sc, std::integral_constant<int, 0>{}, std::true_type{}, std::true_type{},
                      std::false_type{}, before8, after8);
          const StageScales<TM> sc1 = cur_sc;
          mfma_step_x(nxt, sc1, std::integral_constant<int, 1>{}, std::false_type{}, std::true_type{},
                      std::false_type{}, [](int) {}, [&](int k) {
                        between1(k);
                        if (k == 0) pair_store(1, 3);
                      });
        } else if constexpr (MODE == 1) {
          // W4A8, bf16 output: tile k = 4 i + j (i outer) through the staging
          // area after MFMA slot k, its two stores after slot k + 1 (tile 15's
          // after the second step's first MFMA). Rows past M fall past the end
          // of the output (dropped by the range check); columns past N (or no
          // tile at all) get the offset's top bit.
          const i32x4 ry = tile_out(ptm);
          const int ev_m0 = wm * 128 + (lane >> 2);  // row in the tile, + 32 j + 16 st
          const int ev_n0 = ptn * 256 + wn * 128 + (lane & 3) * 8;  // + 32 i
          const uint8_t* prm = ring + PARAM_OFF + ((tile_k - 1) & 1) * PARAM_BYTES;
          float sm[4];  // token scales of the lane's rows, one per row group j
#pragma unroll
          for (int j = 0; j < 4; ++j) sm[j] = *reinterpret_cast<const float*>(prm + P_TOK + (wm * 128 + 32 * j + r) * 4);
          v16f c_cur, c_nxt;
          if constexpr (BIAS) ev_bias(prm, 0, c_cur);
          uint32_t pk[4][2];
          uint4 rd[2];
          auto tile_store = [&](int k) {
            const int i = k >> 2, j = k & 3;
            const uint32_t bad = ev_live && ev_n0 + 32 * i < N ? 0u : 0x80000000u;
#pragma unroll
            for (int st = 0; st < 2; ++st) {
              const uint32_t off = ((uint32_t)(ev_m0 + 32 * j + 16 * st) * (uint32_t)N + (uint32_t)(ev_n0 + 32 * i)) * 2u;
              buf_store16(ry, off | bad, rd[st]);
            }
          };
          auto before8 = [&](int k) {
            const int i = k >> 2, j = k & 3;
            if (BIAS && j == 0 && i > 0) c_cur = c_nxt;
            ev_tile(i, j, c_cur, sm[j], pk);
          };
          auto after8 = [&](int k) {
            const int i = k >> 2, j = k & 3;
            between0(k);
            if (k > 0) tile_store(k - 1);
            ev8_write(pk);
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            ev8_read(rd);
            // the next tile's writes stay behind these reads
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            if (BIAS && j == 1 && i < 3) ev_bias(prm, i + 1, c_nxt);
          };
          mfma_step_x(cur, cur_sc, std::integral_constant<int, 0>{}, std::true_type{}, std::true_type{},
                      std::false_type{}, before8, after8);
          const StageScales<TM> sc1 = cur_sc;
          mfma_step_x(nxt, sc1, std::integral_constant<int, 1>{}, std::false_type{}, std::true_type{},
                      std::false_type{}, [](int) {}, [&](int k) {
                        between1(k);
                        if (k == 0) tile_store(15);
                      });
        } else if constexpr (WAVES == 8) {
          // W4A4, bf16 output, eight waves: tile k = 2 i + j (i outer) through
          // the staging area after MFMA slot k, its two stores of 16 rows x 64
          // bytes after slot k + 1 (tile 7's after the second step's first
          // MFMA), as in the W4A8 epilogue without the token scale. Rows past M
          // fall past the end of the output (dropped by the range check);
          // columns past N (or no tile at all) get the offset's top bit.
          const i32x4 ry = tile_out(ptm);
          const int ev_m0 = wm * 32 * TM + (lane >> 2);  // row in the tile, + 32 j + 16 st
          const int ev_n0 = ptn * 256 + wn * 128 + (lane & 3) * 8;   // + 32 i
          const uint8_t* prm = ring + PARAM_OFF + ((tile_k - 1) & 1) * PARAM_BYTES;
          v16f c_cur, c_nxt;
          if constexpr (BIAS) ev_bias(prm, 0, c_cur);
          uint32_t pk[4][2];
          uint4 rd[2];
          auto tile_store = [&](int k) {
            const int i = k / TM, j = k % TM;
            const uint32_t bad = ev_live && ev_n0 + 32 * i < N ? 0u : 0x80000000u;
#pragma unroll
            for (int st = 0; st < 2; ++st) {
              const uint32_t off = ((uint32_t)(ev_m0 + 32 * j + 16 * st) * (uint32_t)N + (uint32_t)(ev_n0 + 32 * i)) * 2u;
              buf_store16(ry, off | bad, rd[st]);
            }
          };
          auto before8 = [&](int k) {
            const int i = k / TM, j = k % TM;
            if (BIAS && j == 0 && i > 0) c_cur = c_nxt;
            ev_tile(i, j, c_cur, 1.0f, pk);
          };
          auto after8 = [&](int k) {
            const int i = k / TM, j = k % TM;
            between0(k);
            if (k > 0) tile_store(k - 1);
            ev8_write(pk);
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            ev8_read(rd);
            // the next tile's writes stay behind these reads
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            if (BIAS && j == 0 && i < 3) ev_bias(prm, i + 1, c_nxt);
          };
          mfma_step_x(cur, cur_sc, std::integral_constant<int, 0>{}, std::true_type{}, std::true_type{},
                      std::false_type{}, before8, after8);
          const StageScales<TM> sc1 = cur_sc;
          mfma_step_x(nxt, sc1, std::integral_constant<int, 1>{}, std::false_type{}, std::true_type{},
                      std::false_type{}, [](int) {}, [&](int k) {
                        between1(k);
                        if (k == 0) tile_store(NT - 1);
                      });
        } else {
          // byte offset of the lane's first store in the tile's rows (+ 32 j
          // rows + 8 it rows + 64 h columns); rows past M fall past the end of
          // the tile's resource, which the range check drops, and columns past
          // N (or no tile at all) get the offset's top bit, past every tile's
          // rows (256 N 2 bytes < 2^31)
          const i32x4 ry = tile_out(ptm);
          const int ev_m0 = wm * 128 + (lane >> 3);
          const int ev_n0 = ptn * 256 + wn * 128 + (lane & 7) * 8;
          const uint32_t ev_off0 = ((uint32_t)ev_m0 * (uint32_t)N + (uint32_t)ev_n0) * 2u;
          const uint32_t ev_bad0 = ev_live && ev_n0 < N ? 0u : 0x80000000u;
          const uint32_t ev_bad1 = ev_live && ev_n0 + 64 < N ? 0u : 0x80000000u;
          const uint32_t row8 = (uint32_t)N * 16u;  // 8 rows of bf16
          // bias of the finished tile (zeros when there is none)
          const uint8_t* prm = ring + PARAM_OFF + ((tile_k - 1) & 1) * PARAM_BYTES;
          v16f c_cur, c_nxt;
          if constexpr (BIAS) ev_bias(prm, 0, c_cur);
          uint32_t evd[4][4][4][2];
          uint4 rd[4];
          auto unit_store = [&](int j, int h) {
  #pragma unroll
            for (int it = 0; it < 4; ++it)
              buf_store16(ry, (ev_off0 + (uint32_t)(4 * j + it) * row8 + 128u * h) | (h ? ev_bad1 : ev_bad0), rd[it]);
          };
          auto before0 = [&](int k) {
            const int i = k >> 2, j = k & 3;
            if (BIAS && j == 0 && i > 0) c_cur = c_nxt;
            ev_tile(i, j, c_cur, 1.0f, evd[i][j]);
          };
          auto after0 = [&](int k) {
            const int i = k >> 2, j = k & 3;
            between0(k);
            // stores of the pair staged in the previous slot
            if ((k - 1) >> 2 == 1 || (k - 1) >> 2 == 3) unit_store((k - 1) & 3, (k - 1) >> 3);
            if (i & 1) {
              ev_unit_write(evd[i - 1][j], evd[i][j]);
              __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
              ev_unit_read(rd);
              // the next pair's writes stay behind these reads
              __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            }
            if (BIAS && j == 1 && i < 3) ev_bias(prm, i + 1, c_nxt);
          };
          mfma_step_x(cur, cur_sc, std::integral_constant<int, 0>{}, std::true_type{}, std::true_type{},
                      std::false_type{}, before0, after0);
          const StageScales<TM> sc1 = cur_sc;
          mfma_step_x(nxt, sc1, std::integral_constant<int, 1>{}, std::false_type{}, std::true_type{},
                      std::false_type{}, [](int) {}, [&](int k) {
                        between1(k);
                        if (k == 0) unit_store(3, 1);
                      });
        }
      }
      advance_cursor();
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      slot = slot_next;
    };

    // one more first stage after the last tile: it carries that tile's
    // epilogue (its own MFMAs work on zeros); the loop test is the only exit,
    // at the end of an iteration, so no path leaves between a first stage's
    // MFMAs and the stages that use their sums
    for (int tile_k = 0; tile_k <= count; ++tile_k) {
      run_stage(tile_k, 0, std::true_type{}, std::false_type{});
      const int s_end = tile_k < count ? n_stages : 1;
      if constexpr (LRB) {
        // the code stages, then the branch stages (the last of the tile)
        const int q_end = tile_k < count ? nq : 1;
        for (int s_in = 1; s_in < q_end; ++s_in) run_stage(tile_k, s_in, std::false_type{}, std::false_type{});
        for (int s_in = q_end; s_in < s_end; ++s_in) run_stage(tile_k, s_in, std::false_type{}, std::true_type{});
      } else {
        for (int s_in = 1; s_in < s_end; ++s_in) run_stage(tile_k, s_in, std::false_type{}, std::false_type{});
      }
    }
  }
  // no copy or store may still be in flight when the workgroup retires
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
}

// One workgroup per CU (the kernel holds a whole CU's LDS and registers),
// each walking its share of the tiles.
static int device_cu_count() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;
  return cus;
}

template <int MODE, int KT, int NB, int WAVES, int QOUT = 0, bool LRB = false>
static hipError_t launch_pipe(const void* aq, const void* as, const void* wq, const void* ws, const void* bias,
                              int epi, void* y, int64_t M, int64_t N, int64_t K, hipStream_t s,
                              void* y_scales = nullptr, const float* out_amax = nullptr,
                              const void* lr_t = nullptr, const void* lr_l2 = nullptr, int lr_rank = 0,
                              const float* out_mult = nullptr) {
  static const int cus = device_cu_count();
  const int tiles_m = (int)((M + 255) / 256);
  const int tiles_n = (int)((N + 255) / 256);
  const int total = tiles_m * tiles_n;
  const int grid = total < cus ? total : cus;
  // GELU and bias are kernel parameters, so that each kernel carries only
  // the epilogue work it does
  auto go = [&](auto gelu_tag, auto bias_tag) {
    hipLaunchKernelGGL(
        (gemm_pipe_kernel<MODE, KT, NB, decltype(gelu_tag)::value, decltype(bias_tag)::value, QOUT, LRB, WAVES>),
        dim3(grid), dim3(64 * WAVES), 0, s, static_cast<const uint8_t*>(wq), static_cast<const uint8_t*>(ws),
        static_cast<const uint8_t*>(aq), as, static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(y),
        static_cast<uint8_t*>(y_scales), out_amax, (int)M, (int)N, (int)K, tiles_m, tiles_n,
        static_cast<const uint16_t*>(lr_t), static_cast<const uint16_t*>(lr_l2), lr_rank, out_mult);
  };
  if (epi == 1) {
    if (bias != nullptr) go(std::true_type{}, std::true_type{});
    else go(std::true_type{}, std::false_type{});
  } else {
    if (bias != nullptr) go(std::false_type{}, std::true_type{});
    else go(std::false_type{}, std::false_type{});
  }
  return hipGetLastError();
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

// Stage shape of the pipelined kernel per mode: K elements per stage and LDS
// ring depth (chosen from measurements on MI355X). W4A4 runs one wave per SIMD
// (four per workgroup, 128 x 128 outputs each) or two (eight, 128 x 64 each:
// one wave's copies, LDS reads, barrier wait and epilogue overlap the other's
// MFMAs); W4A8, whose ring leaves no room for eight staging areas, and the
// SVDQuant branch stages run one wave per SIMD.
constexpr int kPipeKT[2] = {128, 128};
constexpr int kPipeNB[2] = {4, 3};

// W4A4 wave count per launch. Under sustained load the board holds its power
// cap (1400 W measured on random data) by lowering the clock, and there the
// eight-wave kernel, busier but with 1.5x the LDS reads per MFMA, runs no
// faster than the four-wave one (A14B stack step 1003.6 / 1004.5 ms). Short
// launches finish at a higher clock, where the eight-wave kernel's shorter
// epilogue stage (6.0k against 8.1k cycles) and better overlap pay: 3-4% on
// the TI2V-5B linears, 8% on the 512-token text GEMMs, measured interleaved.
// MXQ_W4A4_WAVES=4 or 8 fixes the choice (read at every call, so tests can
// run either kernel on any shape).
constexpr double kEightWaveMaxFlops = 2e12;
static bool w4a4_eight_waves(int64_t M, int64_t N, int64_t K) {
  const char* v = getenv("MXQ_W4A4_WAVES");
  if (v != nullptr && (v[0] == '4' || v[0] == '8') && v[1] == '\0') return v[0] == '8';
  return 2.0 * (double)M * (double)N * (double)K < kEightWaveMaxFlops;
}

// The pipelined kernel needs whole stages along K, at least NB of them (one
// tile's epilogue is over before the next one starts), and N in multiples of 8
// (16-byte stores); every Wan2.2 linear qualifies. Everything else takes the
// direct kernel. 32-bit buffer offsets, and the out-of-range offset 2^31 that
// must exceed every size, bound every operand below 2^31 bytes; row-major
// outputs are addressed per tile (256 rows: any M), the MXFP4 output as a whole.
static bool use_lds(int mode, int64_t M, int64_t N, int64_t K) {
  const int64_t a_bytes = mode == 0 ? M * (K / 2) : M * K;
  return K % kPipeKT[mode] == 0 && K / kPipeKT[mode] >= kPipeNB[mode] && N % 8 == 0 && M >= 256 && N >= 256 &&
         a_bytes < (int64_t(1) << 31) && N * (K / 2) < (int64_t(1) << 31) && 256 * N * 2 < (int64_t(1) << 31) &&
         M < (int64_t(1) << 31) / 4;
}

// MXFP4 output (codes in panels over all M rows, scales [N/128][M][4]): below 2^31 bytes.
static bool mxfp4_out_fits(int64_t M, int64_t N) { return M * (N / 2) < (int64_t(1) << 31) - 256; }

hipError_t launch_gemm(int mode, const void* a_codes, const void* a_scales,
                       const void* w_codes, const void* w_scales, const void* bias,
                       int epilogue, void* y, int64_t M, int64_t N, int64_t K,
                       hipStream_t s) {
  if (use_lds(mode, M, N, K)) {
    if (mode == 0 && w4a4_eight_waves(M, N, K))
      return launch_pipe<0, kPipeKT[0], kPipeNB[0], 8>(a_codes, a_scales, w_codes, w_scales, bias, epilogue, y, M, N,
                                                       K, s);
    if (mode == 0)
      return launch_pipe<0, kPipeKT[0], kPipeNB[0], 4>(a_codes, a_scales, w_codes, w_scales, bias, epilogue, y, M, N,
                                                       K, s);
    return launch_pipe<1, kPipeKT[1], kPipeNB[1], 4>(a_codes, a_scales, w_codes, w_scales, bias, epilogue, y, M, N,
                                                     K, s);
  }
  if (mode == 0)
    return launch_direct<0, 2, 2>(a_codes, a_scales, w_codes, w_scales, bias, epilogue, y, M, N, K, s);
  return launch_direct<1, 2, 2>(a_codes, a_scales, w_codes, w_scales, bias, epilogue, y, M, N, K, s);
}

bool gemm_mxfp4_out_supported(int64_t M, int64_t N, int64_t K) {
  return use_lds(0, M, N, K) && N % 128 == 0 && mxfp4_out_fits(M, N);
}

hipError_t launch_gemm_mxfp4_out(const void* a_codes, const void* a_scales, const void* w_codes,
                                 const void* w_scales, const void* bias, int epilogue, void* y_codes,
                                 void* y_scales, int64_t M, int64_t N, int64_t K, hipStream_t s) {
  if (w4a4_eight_waves(M, N, K))
    return launch_pipe<0, kPipeKT[0], kPipeNB[0], 8, 1>(a_codes, a_scales, w_codes, w_scales, bias, epilogue,
                                                        y_codes, M, N, K, s, y_scales);
  return launch_pipe<0, kPipeKT[0], kPipeNB[0], 4, 1>(a_codes, a_scales, w_codes, w_scales, bias, epilogue,
                                                      y_codes, M, N, K, s, y_scales);
}

// The transformed output runs on the four-wave kernel at every size (its
// rotated row group needs the registers that the eight-wave kernel's second
// wave takes).
hipError_t launch_gemm_mxfp4_hadamard_out(const void* a_codes, const void* a_scales, const void* w_codes,
                                          const void* w_scales, const void* bias, int epilogue, const float* mult,
                                          void* y_codes, void* y_scales, int64_t M, int64_t N, int64_t K,
                                          hipStream_t s) {
  return launch_pipe<0, kPipeKT[0], kPipeNB[0], 4, 2>(a_codes, a_scales, w_codes, w_scales, bias, epilogue,
                                                      y_codes, M, N, K, s, y_scales, nullptr, nullptr, nullptr, 0,
                                                      mult);
}

// N is the next layer's K: a multiple of 32
bool gemm_fp8_static_out_supported(int64_t M, int64_t N, int64_t K) { return use_lds(1, M, N, K) && N % 32 == 0; }

hipError_t launch_gemm_fp8_static_out(const void* a_codes, const void* a_scales, const void* w_codes,
                                      const void* w_scales, const void* bias, int epilogue, const float* out_amax,
                                      void* y_codes, void* y_scales, int64_t M, int64_t N, int64_t K,
                                      hipStream_t s) {
  return launch_pipe<1, kPipeKT[1], kPipeNB[1], 4, 1>(a_codes, a_scales, w_codes, w_scales, bias, epilogue,
                                                      y_codes, M, N, K, s, y_scales, out_amax);
}

// The branch rides on the pipelined W4A4 kernel (its shapes only); with
// y_scales the output is MXFP4 as for launch_gemm_mxfp4_out (N % 128 == 0).
bool gemm_lowrank_supported(int64_t M, int64_t N, int64_t K, bool mxfp4_out) {
  return use_lds(0, M, N, K) && (!mxfp4_out || (N % 128 == 0 && mxfp4_out_fits(M, N)));
}

hipError_t launch_gemm_lowrank(const void* a_codes, const void* a_scales, const void* w_codes,
                               const void* w_scales, const void* bias, const void* t, const void* l2, int64_t r,
                               int epilogue, void* y, void* y_scales, int64_t M, int64_t N, int64_t K,
                               hipStream_t s) {
  if (y_scales != nullptr)
    return launch_pipe<0, kPipeKT[0], kPipeNB[0], 4, 1, true>(a_codes, a_scales, w_codes, w_scales, bias,
                                                              epilogue, y, M, N, K, s, y_scales, nullptr, t, l2,
                                                              (int)r);
  return launch_pipe<0, kPipeKT[0], kPipeNB[0], 4, 0, true>(a_codes, a_scales, w_codes, w_scales, bias, epilogue,
                                                             y, M, N, K, s, nullptr, nullptr, t, l2, (int)r);
}

const char* gemm_variant_name(int mode, int64_t M, int64_t N, int64_t K) {
  if (use_lds(mode, M, N, K))
    return mode == 0 ? (w4a4_eight_waves(M, N, K) ? "pipe_w4a4_wg256x256_wave128x64" : "pipe_w4a4_wg256x256_wave128x128")
                     : "pipe_w4a8_wg256x256_wave128x128";
  return mode == 0 ? "direct_w4a4_wg128x128_wave64x64" : "direct_w4a8_wg128x128_wave64x64";
}

}  // namespace mxq
