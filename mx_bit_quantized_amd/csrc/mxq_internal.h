// mxq_internal.h - launchers shared between the C ABI layer and the kernels.
// Callers have validated every argument; launchers only enqueue work.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

// MXFP4 quantizer; `weight` selects the kernel instance that offline weight
// packing runs under (same code, its own symbol in profiles).
hipError_t launch_mxfp4_quant(const void* x, int64_t rows, int64_t K, int64_t ld,
                              void* codes, void* scales, hipStream_t s, bool weight = false);

hipError_t launch_fp8_quant(const void* x, int64_t rows, int64_t K, int64_t ld,
                            void* codes, void* scales, hipStream_t s);

// transform_on: MXFP4 codes and scales of RN_bf16(hadamard128(x) * mult)
// (K % 128 == 0); the per-channel rotated amax for SmoothQuant calibration
// (running maximum, amax [K]); the SmoothQuant factor vectors from two of them.
hipError_t launch_mxfp4_hadamard_quant(const void* x, int64_t rows, int64_t K, int64_t ld, const float* mult,
                                       void* codes, void* scales, hipStream_t s);
hipError_t launch_hadamard_amax(const void* x, int64_t rows, int64_t K, int64_t ld, float* amax, hipStream_t s);
hipError_t launch_smoothquant_factors(const float* act_amax, const float* w_amax, int64_t K, float* act_mult,
                                      float* w_mult, hipStream_t s);

// SVDQuant's low-rank branch: t [M][r] = RN_bf16(x L1) from l1t [r][K]
// (r = 32, 64, 96 or 128; K % 128 == 0); y [M][N] = RN_bf16(epilogue(y_pre +
// t L2^T)) from l2 [N][r] (N % 32 == 0; y may be y_pre).
// t = RN_bf16(x l1t^T); with codes non-null also the W4A4 activation of x
// (codes in 128-element panels, scales [K/128][M][4]) in the same pass.
hipError_t launch_lowrank_down(const void* x, int64_t M, int64_t K, const void* l1t, int64_t r, void* t,
                               void* codes, void* scales, hipStream_t s);
hipError_t launch_lowrank_up(const void* y_pre, const void* t, const void* l2, int64_t M, int64_t N, int64_t r,
                             int epilogue, void* y, hipStream_t s);

// Block selection: sums[0] += sum r^2, sums[1] += sum (y - r)^2 over n bf16
// elements (fp64, device [2]); a zero fill of n 4-byte words.
hipError_t launch_sqnr_sums(const void* y, const void* y_ref, int64_t n, double* sums, hipStream_t s);
hipError_t launch_fill_zero(void* p, int64_t n_words, hipStream_t s);

// Static FP8: codes with the one scale amax / 448 (amax: device fp32), every
// row's scale slot set to it.
hipError_t launch_fp8_static_quant(const void* x, int64_t rows, int64_t K, int64_t ld, const float* amax,
                                   void* codes, void* scales, hipStream_t s);

// *amax = max(*amax, max |x|) over a [rows, K] bf16 matrix (device fp32, >= 0).
hipError_t launch_fp8_amax(const void* x, int64_t rows, int64_t K, int64_t ld, float* amax, hipStream_t s);

// y[M][N] = epilogue(A * W^T + bias); mode 0 = W4A4, 1 = W4A8.
hipError_t launch_gemm(int mode, const void* a_codes, const void* a_scales,
                       const void* w_codes, const void* w_scales, const void* bias,
                       int epilogue, void* y, int64_t M, int64_t N, int64_t K,
                       hipStream_t s);

// W4A4 GEMM whose bf16 output goes straight into the MXFP4 activation
// format (codes in code panels along N, scales [N/128][M][4]); only for shapes
// where gemm_mxfp4_out_supported holds.
bool gemm_mxfp4_out_supported(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_mxfp4_out(const void* a_codes, const void* a_scales, const void* w_codes,
                                 const void* w_scales, const void* bias, int epilogue, void* y_codes,
                                 void* y_scales, int64_t M, int64_t N, int64_t K, hipStream_t s);

// The same with the transform_on rotation of the output before MXFP4: the
// codes and scales of launch_mxfp4_hadamard_quant(bf16 output, mult), mult
// device float [N].
hipError_t launch_gemm_mxfp4_hadamard_out(const void* a_codes, const void* a_scales, const void* w_codes,
                                          const void* w_scales, const void* bias, int epilogue, const float* mult,
                                          void* y_codes, void* y_scales, int64_t M, int64_t N, int64_t K,
                                          hipStream_t s);

// W4A8 GEMM whose bf16 output goes straight into static FP8 with the scale
// out_amax / 448 (device fp32): codes [M][N], the scale in every row of
// y_scales (float [M]); only where gemm_fp8_static_out_supported holds.
bool gemm_fp8_static_out_supported(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_fp8_static_out(const void* a_codes, const void* a_scales, const void* w_codes,
                                      const void* w_scales, const void* bias, int epilogue, const float* out_amax,
                                      void* y_codes, void* y_scales, int64_t M, int64_t N, int64_t K,
                                      hipStream_t s);

// W4A4 GEMM with SVDQuant's branch t [M][r] l2[N][r]^T in its fp32 sums,
// bf16 output (y_scales null) or MXFP4 output as launch_gemm_mxfp4_out; only
// where gemm_lowrank_supported holds.
bool gemm_lowrank_supported(int64_t M, int64_t N, int64_t K, bool mxfp4_out);
hipError_t launch_gemm_lowrank(const void* a_codes, const void* a_scales, const void* w_codes,
                               const void* w_scales, const void* bias, const void* t, const void* l2, int64_t r,
                               int epilogue, void* y, void* y_scales, int64_t M, int64_t N, int64_t K,
                               hipStream_t s);

// MXFP4 codes and scales between the library layout (code panels, group-major
// scales) and the canonical row-major one ([rows][K/2], [rows][K/32]).
hipError_t launch_mxfp4_layout(bool to_canonical, const void* src_codes, const void* src_scales, int64_t rows,
                               int64_t K, void* dst_codes, void* dst_scales, hipStream_t s);

// The optional non-finite guard: whether MXQ_CHECK_FINITE is set, and a scan
// of a bf16 [rows][ld] matrix's first cols columns (synchronizes the stream;
// *found tells whether a value is infinite or NaN; returns nonzero on a HIP
// error).
bool check_finite_enabled();
int scan_nonfinite_bf16(const void* x, int64_t rows, int64_t cols, int64_t ld, hipStream_t s, bool* found);

// Name of the GEMM kernel variant launch_gemm picks for a shape (for logs).
const char* gemm_variant_name(int mode, int64_t M, int64_t N, int64_t K);

}  // namespace mxq
