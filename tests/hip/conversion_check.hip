// Exhaustive GPU checks of the gfx950 conversion instructions the quantizers
// use, against the software rounding in mxq_convert.h (whose host build is
// checked exhaustively against the CPU oracle). Test infrastructure only.
//
//   mxq_check_fp4(counts, first): v_cvt_scalef32_pk_fp4_bf16 with the scale
//     byte in the fp32 exponent field, against e2m1_code_bf16, for every
//     finite bf16 and every scale byte 0..252 of a block that can hold it
//     (|v| 2^-E < 8), both nibbles of the packed result.
//   mxq_check_fp8(counts, first): v_cvt_pk_fp8_f32 against e4m3fn_code for
//     every fp32 with |q| <= 464 (the quotients of the FP8 quantizer stay
//     below 448 (1 + 2^-22)), both signs.
//   mxq_check_bf16(counts, first): v_cvt_pk_bf16_f32 against bf16_rne for
//     every non-NaN fp32 (infinities, subnormals and zeros included), both
//     signs (the transformed MXFP4 quantizer rounds its fp32 values with it).
// counts[0] receives the number of mismatches, counts[1] the number of cases;
// first[] the first (input, reference, result) triples. Returns 0, or 1/2 on
// a HIP error.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq_convert.h"

using namespace mxq;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ void note(unsigned long long* counts, uint32_t* first, uint32_t a, uint32_t b, uint32_t c) {
  const unsigned long long n = atomicAdd(&counts[0], 1ull);
  if (n < 8) {
    first[3 * n] = a;
    first[3 * n + 1] = b;
    first[3 * n + 2] = c;
  }
}

__global__ void fp4_kernel(unsigned long long* counts, uint32_t* first) {
  const uint32_t idx = blockIdx.x * 256u + threadIdx.x;  // (bits16 << 8) | scale byte
  const uint32_t bits = idx >> 8, sb = idx & 255u;
  const uint32_t mag = bits & 0x7FFFu;
  const int e_field = (int)(mag >> 7);
  // finite, a valid scale byte, and |v| 2^-E < 8 (v can sit in a block of that scale)
  const bool live = sb <= 252u && (bits & 0x7F80u) != 0x7F80u && !(e_field > 0 && e_field - (int)sb >= 3);
  const int n_live = __syncthreads_count(live);
  if (threadIdx.x == 0) atomicAdd(&counts[1], (unsigned long long)n_live);
  if (!live) return;
  const uint32_t ref = e2m1_code_bf16(bits, mx_inv_scale(sb));
  const uint32_t other = (bits ^ 0x8000u);  // the opposite sign in the high half
  const uint32_t ref_hi = e2m1_code_bf16(other, mx_inv_scale(sb));
  const bf16x2_t v = __builtin_bit_cast(bf16x2_t, bits | (other << 16));
  const uint32_t hw = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, v, as_float(sb << 23), 0) & 0xFFu;
  if (hw != (ref | (ref_hi << 4))) note(counts, first, idx, ref | (ref_hi << 4), hw);
}

__global__ void fp8_kernel(unsigned long long* counts, uint32_t* first, uint32_t limit) {
  const uint32_t a = blockIdx.x * 256u + threadIdx.x;
  const bool live = a <= limit;
  const int n_live = __syncthreads_count(live);
  if (threadIdx.x == 0) atomicAdd(&counts[1], 2ull * (unsigned long long)n_live);
  if (!live) return;
  const float q = as_float(a), nq = as_float(a | 0x80000000u);
  const uint32_t ref = e4m3fn_code(q) | (e4m3fn_code(nq) << 8);
  const uint32_t hw = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q, nq, 0, false) & 0xFFFFu;
  if (hw != ref) note(counts, first, a, ref, hw);
}

typedef float v2f_t __attribute__((ext_vector_type(2)));

__global__ void bf16_kernel(unsigned long long* counts, uint32_t* first) {
  const uint32_t a = blockIdx.x * 256u + threadIdx.x;  // every pattern with the sign bit clear
  const bool live = a <= 0x7F800000u;                   // not NaN
  const int n_live = __syncthreads_count(live);
  if (threadIdx.x == 0) atomicAdd(&counts[1], 2ull * (unsigned long long)n_live);
  if (!live) return;
  const float q = as_float(a), nq = as_float(a | 0x80000000u);
  const uint32_t ref = bf16_rne(q) | (bf16_rne(nq) << 16);
  const v2f_t f = {q, nq};
  const uint32_t hw = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
  if (hw != ref) note(counts, first, a, ref, hw);
}

static int finish(unsigned long long* d_counts, uint32_t* d_first, unsigned long long* counts, uint32_t* first) {
  if (hipDeviceSynchronize() != hipSuccess) return 2;
  if (hipMemcpy(counts, d_counts, 16, hipMemcpyDeviceToHost) != hipSuccess) return 2;
  if (hipMemcpy(first, d_first, 24 * 4, hipMemcpyDeviceToHost) != hipSuccess) return 2;
  (void)hipFree(d_counts);
  (void)hipFree(d_first);
  return 0;
}

static int setup(unsigned long long** d_counts, uint32_t** d_first) {
  if (hipMalloc(d_counts, 16) != hipSuccess || hipMalloc(d_first, 24 * 4) != hipSuccess) return 1;
  if (hipMemset(*d_counts, 0, 16) != hipSuccess || hipMemset(*d_first, 0, 24 * 4) != hipSuccess) return 1;
  return 0;
}

extern "C" int mxq_check_fp4(unsigned long long* counts, uint32_t* first) {
  unsigned long long* dc;
  uint32_t* df;
  if (setup(&dc, &df)) return 1;
  hipLaunchKernelGGL(fp4_kernel, dim3(65536), dim3(256), 0, 0, dc, df);
  if (hipGetLastError() != hipSuccess) return 1;
  return finish(dc, df, counts, first);
}

extern "C" int mxq_check_fp8(unsigned long long* counts, uint32_t* first) {
  unsigned long long* dc;
  uint32_t* df;
  if (setup(&dc, &df)) return 1;
  const uint32_t limit = 0x43E80000u;  // 464.0f
  hipLaunchKernelGGL(fp8_kernel, dim3(limit / 256u + 1u), dim3(256), 0, 0, dc, df, limit);
  if (hipGetLastError() != hipSuccess) return 1;
  return finish(dc, df, counts, first);
}

extern "C" int mxq_check_bf16(unsigned long long* counts, uint32_t* first) {
  unsigned long long* dc;
  uint32_t* df;
  if (setup(&dc, &df)) return 1;
  hipLaunchKernelGGL(bf16_kernel, dim3(0x80000000u / 256u), dim3(256), 0, 0, dc, df);
  if (hipGetLastError() != hipSuccess) return 1;
  return finish(dc, df, counts, first);
}
