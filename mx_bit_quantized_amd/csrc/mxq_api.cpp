// mxq_api.cpp - the extern "C" boundary of libmxq (declared in include/mxq.h).
//
// Host-side validation, the per-expert / per-block policy table of section
// "Practical workflow" (step 6) of the page "Quark Mixed-Precision
// Quantization for Wan2.2 Video Generation on AMD Instinct GPUs", and dispatch
// to the gfx950 kernels. Every check runs before anything is enqueued, so a
// failing call writes nothing; modes other than W4A4 / W4A8 are errors, never
// a silent fallback.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <math.h>

#include <new>
#include <vector>

#include "mxq.h"
#include "mxq_internal.h"

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;

struct Policy {
  int32_t n_experts;
  int32_t n_blocks;
  std::vector<uint8_t> modes;
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool log_enabled() {
  static const int on = [] {
    const char* v = getenv("MXQ_LOG");
    return (v != nullptr && v[0] != '\0' && v[0] != '0') ? 1 : 0;
  }();
  return on != 0;
}

int check_mk(int64_t rows, int64_t K, int64_t ld) {
  if (rows < 0 || K <= 0 || ld < 0) return MXQ_ERR_SHAPE;
  if (K % 32 != 0 || ld < K) return MXQ_ERR_SHAPE;
  if (rows >= kMaxDim || K >= kMaxDim || ld >= kMaxDim) return MXQ_ERR_SHAPE;
  return MXQ_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MXQ_OK : MXQ_ERR_HIP; }

// MXQ_CHECK_FINITE: scan a bf16 [rows][ld] input (or output) for infinities and
// NaNs; MXQ_OK when the guard is off.
int finite_guard(const char* what, const void* x, int64_t rows, int64_t cols, int64_t ld, hipStream_t stream) {
  if (!mxq::check_finite_enabled()) return MXQ_OK;
  bool bad = false;
  if (mxq::scan_nonfinite_bf16(x, rows, cols, ld, stream, &bad) != 0) return MXQ_ERR_HIP;
  if (!bad) return MXQ_OK;
  if (log_enabled()) fprintf(stderr, "[mxq] non-finite value in %s [%lld x %lld]\n", what, (long long)rows,
                             (long long)cols);
  return MXQ_ERR_NONFINITE;
}

// a launch's status, then the guard on its bf16 output
int output_guard(hipError_t e, const char* what, const void* y, int64_t rows, int64_t cols, hipStream_t stream) {
  if (e != hipSuccess) return MXQ_ERR_HIP;
  return finite_guard(what, y, rows, cols, cols, stream);
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace layout of mxq_qlinear: codes first, scales at a 256-byte boundary.
void workspace_layout(int mode, int64_t M, int64_t K, size_t* codes_bytes, size_t* total) {
  size_t cb = mode == MXQ_W4A4 ? (size_t)M * (size_t)(K / 2) : (size_t)M * (size_t)K;
  size_t sb = mode == MXQ_W4A4 ? (size_t)M * 4 * (size_t)((K + 127) / 128) : (size_t)M * sizeof(float);
  *codes_bytes = round_up(cb, 256);
  *total = *codes_bytes + round_up(sb, 256);
}

// Workspace layout of mxq_block_replay_sqnr for one linear: activation codes
// and scales, weight codes and scales (W4A4 layouts), y (bf16), then four fp32
// vectors of K (x maxima, w maxima, act factors, w factors); 256-byte aligned.
struct ReplayLayout {
  size_t a_codes, a_scales, w_codes, w_scales, y, ax, aw, am, wm, total;
};

ReplayLayout replay_layout(int64_t M, int64_t N, int64_t K) {
  ReplayLayout L{};
  size_t cb = 0, tot = 0, off = 0;
  workspace_layout(MXQ_W4A4, M, K, &cb, &tot);
  L.a_codes = off;
  L.a_scales = off + cb;
  off += tot;
  workspace_layout(MXQ_W4A4, N, K, &cb, &tot);
  L.w_codes = off;
  L.w_scales = off + cb;
  off += tot;
  L.y = off;
  off += round_up((size_t)M * (size_t)N * 2, 256);
  const size_t kv = round_up((size_t)K * 4, 256);
  L.ax = off;
  L.aw = off + kv;
  L.am = off + 2 * kv;
  L.wm = off + 3 * kv;
  L.total = off + 4 * kv;
  return L;
}

int check_replay_linear(const mxq_replay_linear& l) {
  int st = check_mk(l.M, l.K, l.K);
  if (st != MXQ_OK) return st;
  if (l.M < 1 || l.N < 1 || l.N >= kMaxDim || l.K % 128 != 0) return MXQ_ERR_SHAPE;
  if (l.x == nullptr || l.w == nullptr || l.y_ref == nullptr) return MXQ_ERR_NULL;
  if (!aligned16(l.x) || !aligned16(l.w) || !aligned16(l.y_ref)) return MXQ_ERR_ALIGN;
  return MXQ_OK;
}

double sqnr_of(const double* sums) {
  if (sums[1] == 0.0) return INFINITY;
  if (sums[0] == 0.0) return -INFINITY;
  return 10.0 * log10(sums[0] / sums[1]);
}

}  // namespace

extern "C" {

const char* mxq_status_string(int status) {
  switch (status) {
    case MXQ_OK: return "ok";
    case MXQ_ERR_NULL: return "null pointer";
    case MXQ_ERR_SHAPE: return "bad shape (sizes must be >= 0, K a positive multiple of 32, ld >= K, dims < 2^31)";
    case MXQ_ERR_ALIGN: return "misaligned (device pointers need 16-byte alignment, ld a multiple of 8)";
    case MXQ_ERR_MODE: return "unsupported mode or epilogue (quantized linear modes are W4A4 and W4A8)";
    case MXQ_ERR_WORKSPACE: return "workspace missing or too small";
    case MXQ_ERR_HIP: return "HIP launch or runtime error";
    case MXQ_ERR_RANGE: return "policy index out of range";
    case MXQ_ERR_SCRATCH: return "problem too large for the allocation-free scratch area (64 MiB)";
    case MXQ_ERR_NONFINITE: return "non-finite value (infinity or NaN) in an input or output (MXQ_CHECK_FINITE)";
    default: return "unknown status";
  }
}

int mxq_version(void) { return 10100; }

int mxq_quantize_weight_mxfp4(const void* w, int64_t N, int64_t K, int64_t ldw,
                              void* codes, void* scales, hipStream_t stream) {
  int st = check_mk(N, K, ldw);
  if (st != MXQ_OK) return st;
  if (N == 0) return MXQ_OK;
  if (w == nullptr || codes == nullptr || scales == nullptr) return MXQ_ERR_NULL;
  if (!aligned16(w) || !aligned16(codes) || !aligned16(scales) || ldw % 8 != 0) return MXQ_ERR_ALIGN;
  if (log_enabled()) fprintf(stderr, "[mxq] quantize_weight_mxfp4 N=%lld K=%lld\n", (long long)N, (long long)K);
  if ((st = finite_guard("weight", w, N, K, ldw, stream)) != MXQ_OK) return st;
  return hip_status(mxq::launch_mxfp4_quant(w, N, K, ldw, codes, scales, stream, true));
}

int mxq_quantize_act(int mode, const void* x, int64_t M, int64_t K, int64_t ldx,
                     void* codes, void* scales, hipStream_t stream) {
  if (mode != MXQ_W4A4 && mode != MXQ_W4A8) return MXQ_ERR_MODE;
  int st = check_mk(M, K, ldx);
  if (st != MXQ_OK) return st;
  if (M == 0) return MXQ_OK;
  if (x == nullptr || codes == nullptr || scales == nullptr) return MXQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales) || ldx % 8 != 0) return MXQ_ERR_ALIGN;
  if (log_enabled())
    fprintf(stderr, "[mxq] quantize_act %s M=%lld K=%lld\n", mode == MXQ_W4A4 ? "mxfp4" : "fp8_per_token",
            (long long)M, (long long)K);
  if ((st = finite_guard("activation", x, M, K, ldx, stream)) != MXQ_OK) return st;
  if (mode == MXQ_W4A4) return hip_status(mxq::launch_mxfp4_quant(x, M, K, ldx, codes, scales, stream));
  return hip_status(mxq::launch_fp8_quant(x, M, K, ldx, codes, scales, stream));
}

int mxq_hadamard_channel_amax(const void* x, int64_t M, int64_t K, int64_t ldx, float* amax, hipStream_t stream) {
  int st = check_mk(M, K, ldx);
  if (st != MXQ_OK) return st;
  if (K % 128 != 0) return MXQ_ERR_SHAPE;
  if (M == 0) return MXQ_OK;
  if (x == nullptr || amax == nullptr) return MXQ_ERR_NULL;
  if (!aligned16(x) || ldx % 8 != 0 || (reinterpret_cast<uintptr_t>(amax) & 3u) != 0) return MXQ_ERR_ALIGN;
  if (log_enabled()) fprintf(stderr, "[mxq] hadamard_channel_amax M=%lld K=%lld\n", (long long)M, (long long)K);
  if ((st = finite_guard("calibration input", x, M, K, ldx, stream)) != MXQ_OK) return st;
  return hip_status(mxq::launch_hadamard_amax(x, M, K, ldx, amax, stream));
}

int mxq_smoothquant_factors(const float* act_amax, const float* w_amax, int64_t K, float* act_mult,
                            float* w_mult, hipStream_t stream) {
  if (K < 0 || K >= kMaxDim) return MXQ_ERR_SHAPE;
  if (K == 0) return MXQ_OK;
  if (act_amax == nullptr || w_amax == nullptr || act_mult == nullptr || w_mult == nullptr) return MXQ_ERR_NULL;
  for (const void* p : {(const void*)act_amax, (const void*)w_amax, (const void*)act_mult, (const void*)w_mult})
    if ((reinterpret_cast<uintptr_t>(p) & 3u) != 0) return MXQ_ERR_ALIGN;
  return hip_status(mxq::launch_smoothquant_factors(act_amax, w_amax, K, act_mult, w_mult, stream));
}

int mxq_quantize_mxfp4_hadamard(const void* x, int64_t M, int64_t K, int64_t ldx, const float* mult,
                                void* codes, void* scales, hipStream_t stream) {
  int st = check_mk(M, K, ldx);
  if (st != MXQ_OK) return st;
  if (K % 128 != 0) return MXQ_ERR_SHAPE;
  if (M == 0) return MXQ_OK;
  if (x == nullptr || mult == nullptr || codes == nullptr || scales == nullptr) return MXQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(mult) || !aligned16(codes) || !aligned16(scales) || ldx % 8 != 0)
    return MXQ_ERR_ALIGN;
  if (log_enabled()) fprintf(stderr, "[mxq] quantize_mxfp4_hadamard M=%lld K=%lld\n", (long long)M, (long long)K);
  if ((st = finite_guard("activation", x, M, K, ldx, stream)) != MXQ_OK) return st;
  return hip_status(mxq::launch_mxfp4_hadamard_quant(x, M, K, ldx, mult, codes, scales, stream));
}

static bool lowrank_rank_ok(int64_t r) { return r == 32 || r == 64 || r == 96 || r == 128; }

int mxq_lowrank_down(const void* x, int64_t M, int64_t K, const void* l1t, int64_t r, void* t, hipStream_t stream) {
  int st = check_mk(M, K, K);
  if (st != MXQ_OK) return st;
  if (K % 128 != 0 || !lowrank_rank_ok(r)) return MXQ_ERR_SHAPE;
  if (M == 0) return MXQ_OK;
  if (x == nullptr || l1t == nullptr || t == nullptr) return MXQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(l1t) || !aligned16(t)) return MXQ_ERR_ALIGN;
  if ((st = finite_guard("activation", x, M, K, K, stream)) != MXQ_OK) return st;
  return hip_status(mxq::launch_lowrank_down(x, M, K, l1t, r, t, nullptr, nullptr, stream));
}

int mxq_quantize_act_lowrank(const void* x, int64_t M, int64_t K, const void* l1t, int64_t r, void* codes,
                             void* scales, void* t, hipStream_t stream) {
  int st = check_mk(M, K, K);
  if (st != MXQ_OK) return st;
  if (K % 128 != 0 || !lowrank_rank_ok(r)) return MXQ_ERR_SHAPE;
  if (M == 0) return MXQ_OK;
  if (x == nullptr || l1t == nullptr || codes == nullptr || scales == nullptr || t == nullptr) return MXQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(l1t) || !aligned16(codes) || !aligned16(scales) || !aligned16(t))
    return MXQ_ERR_ALIGN;
  if ((st = finite_guard("activation", x, M, K, K, stream)) != MXQ_OK) return st;
  return hip_status(mxq::launch_lowrank_down(x, M, K, l1t, r, t, codes, scales, stream));
}

int mxq_lowrank_up(const void* y_pre, const void* t, const void* l2, int64_t M, int64_t N, int64_t r,
                   int epilogue, void* y, hipStream_t stream) {
  if (epilogue != MXQ_EPI_NONE && epilogue != MXQ_EPI_GELU_TANH) return MXQ_ERR_MODE;
  if (M < 0 || N < 0 || M >= kMaxDim || N >= kMaxDim || N % 32 != 0 || !lowrank_rank_ok(r)) return MXQ_ERR_SHAPE;
  if (M == 0 || N == 0) return MXQ_OK;
  if (y_pre == nullptr || t == nullptr || l2 == nullptr || y == nullptr) return MXQ_ERR_NULL;
  if (!aligned16(y_pre) || !aligned16(t) || !aligned16(l2) || !aligned16(y)) return MXQ_ERR_ALIGN;
  return output_guard(mxq::launch_lowrank_up(y_pre, t, l2, M, N, r, epilogue, y, stream), "output", y, M, N, stream);
}

int mxq_gemm_lowrank(const void* a_codes, const void* a_scales, const void* w_codes, const void* w_scales,
                     const void* bias, const void* t, const void* l2, int64_t r, int epilogue, void* y,
                     void* y_scales, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  if (epilogue != MXQ_EPI_NONE && epilogue != MXQ_EPI_GELU_TANH) return MXQ_ERR_MODE;
  int st = check_mk(M, K, K);
  if (st != MXQ_OK) return st;
  if (N < 0 || N >= kMaxDim || !lowrank_rank_ok(r)) return MXQ_ERR_SHAPE;
  if (M == 0 || N == 0) return MXQ_OK;
  if (!mxq::gemm_lowrank_supported(M, N, K, y_scales != nullptr)) return MXQ_ERR_SHAPE;
  if (a_codes == nullptr || a_scales == nullptr || w_codes == nullptr || w_scales == nullptr || t == nullptr ||
      l2 == nullptr || y == nullptr)
    return MXQ_ERR_NULL;
  if (!aligned16(a_codes) || !aligned16(a_scales) || !aligned16(w_codes) || !aligned16(w_scales) ||
      !aligned16(t) || !aligned16(l2) || !aligned16(y) || (y_scales != nullptr && !aligned16(y_scales)) ||
      (bias != nullptr && !aligned16(bias)))
    return MXQ_ERR_ALIGN;
  if (log_enabled())
    fprintf(stderr, "[mxq] gemm w4a4 + rank-%lld branch%s M=%lld N=%lld K=%lld epi=%d\n", (long long)r,
            y_scales != nullptr ? " -> mxfp4" : "", (long long)M, (long long)N, (long long)K, epilogue);
  const hipError_t e = mxq::launch_gemm_lowrank(a_codes, a_scales, w_codes, w_scales, bias, t, l2, r, epilogue, y,
                                                y_scales, M, N, K, stream);
  if (y_scales != nullptr) return hip_status(e);  // MXFP4 output: always finite
  return output_guard(e, "output", y, M, N, stream);
}

int mxq_sqnr_accumulate(const void* y, const void* y_ref, int64_t n, double* sums, hipStream_t stream) {
  if (n < 0) return MXQ_ERR_SHAPE;
  if (n == 0) return MXQ_OK;
  if (y == nullptr || y_ref == nullptr || sums == nullptr) return MXQ_ERR_NULL;
  if (!aligned16(y) || !aligned16(y_ref) || (reinterpret_cast<uintptr_t>(sums) & 7u) != 0) return MXQ_ERR_ALIGN;
  return hip_status(mxq::launch_sqnr_sums(y, y_ref, n, sums, stream));
}

int mxq_replay_workspace_bytes(const mxq_replay_linear* linears, int32_t n_linears, size_t* bytes) {
  if (bytes == nullptr) return MXQ_ERR_NULL;
  if (n_linears < 0) return MXQ_ERR_SHAPE;
  if (n_linears > 0 && linears == nullptr) return MXQ_ERR_NULL;
  size_t need = 0;
  for (int32_t i = 0; i < n_linears; ++i) {
    const mxq_replay_linear& l = linears[i];
    if (check_mk(l.M, l.K, l.K) != MXQ_OK || l.M < 1 || l.N < 1 || l.N >= kMaxDim || l.K % 128 != 0)
      return MXQ_ERR_SHAPE;
    const size_t t = replay_layout(l.M, l.N, l.K).total;
    need = t > need ? t : need;
  }
  *bytes = need;
  return MXQ_OK;
}

int mxq_block_replay_sqnr(const mxq_replay_linear* linears, int32_t n_linears, void* workspace,
                          size_t workspace_bytes, double* sums_off, double* sums_on, hipStream_t stream) {
  if (n_linears < 0) return MXQ_ERR_SHAPE;
  if (n_linears == 0) return MXQ_OK;
  if (linears == nullptr || sums_off == nullptr || sums_on == nullptr) return MXQ_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(sums_off) & 7u) != 0 || (reinterpret_cast<uintptr_t>(sums_on) & 7u) != 0)
    return MXQ_ERR_ALIGN;
  size_t need = 0;
  for (int32_t i = 0; i < n_linears; ++i) {
    const int st = check_replay_linear(linears[i]);
    if (st != MXQ_OK) return st;
  }
  int st = mxq_replay_workspace_bytes(linears, n_linears, &need);
  if (st != MXQ_OK) return st;
  if (workspace == nullptr || workspace_bytes < need) return MXQ_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return MXQ_ERR_ALIGN;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  for (int32_t i = 0; i < n_linears; ++i) {
    const mxq_replay_linear& l = linears[i];
    const ReplayLayout L = replay_layout(l.M, l.N, l.K);
    void* ac = ws + L.a_codes;
    void* as = ws + L.a_scales;
    void* wc = ws + L.w_codes;
    void* wsc = ws + L.w_scales;
    void* y = ws + L.y;
    float* ax = reinterpret_cast<float*>(ws + L.ax);
    float* aw = reinterpret_cast<float*>(ws + L.aw);
    float* am = reinterpret_cast<float*>(ws + L.am);
    float* wm = reinterpret_cast<float*>(ws + L.wm);
    const int64_t n_out = l.M * l.N;
    // OFF: plain dynamic MXFP4
    if ((st = mxq_quantize_act(MXQ_W4A4, l.x, l.M, l.K, l.K, ac, as, stream)) != MXQ_OK) return st;
    if ((st = mxq_quantize_weight_mxfp4(l.w, l.N, l.K, l.K, wc, wsc, stream)) != MXQ_OK) return st;
    if ((st = mxq_gemm(MXQ_W4A4, ac, as, wc, wsc, nullptr, MXQ_EPI_NONE, y, l.M, l.N, l.K, stream)) != MXQ_OK)
      return st;
    if ((st = mxq_sqnr_accumulate(y, l.y_ref, n_out, sums_off, stream)) != MXQ_OK) return st;
    // ON: the transform calibrated on this input and weight
    if ((st = hip_status(mxq::launch_fill_zero(ax, 2 * ((L.aw - L.ax) / 4), stream))) != MXQ_OK) return st;
    if ((st = mxq_hadamard_channel_amax(l.x, l.M, l.K, l.K, ax, stream)) != MXQ_OK) return st;
    if ((st = mxq_hadamard_channel_amax(l.w, l.N, l.K, l.K, aw, stream)) != MXQ_OK) return st;
    if ((st = mxq_smoothquant_factors(ax, aw, l.K, am, wm, stream)) != MXQ_OK) return st;
    if ((st = mxq_quantize_mxfp4_hadamard(l.x, l.M, l.K, l.K, am, ac, as, stream)) != MXQ_OK) return st;
    if ((st = mxq_quantize_mxfp4_hadamard(l.w, l.N, l.K, l.K, wm, wc, wsc, stream)) != MXQ_OK) return st;
    if ((st = mxq_gemm(MXQ_W4A4, ac, as, wc, wsc, nullptr, MXQ_EPI_NONE, y, l.M, l.N, l.K, stream)) != MXQ_OK)
      return st;
    if ((st = mxq_sqnr_accumulate(y, l.y_ref, n_out, sums_on, stream)) != MXQ_OK) return st;
  }
  return MXQ_OK;
}

int mxq_policy_select(const double* sums_off, const double* sums_on, int32_t n_experts, int32_t n_blocks,
                      int32_t tier, uint8_t* modes) {
  static const double kTiers[3][3] = {{8.0, 21.0, 0.5}, {10.0, 23.0, 0.5}, {12.0, 25.0, 0.5}};
  if (tier < MXQ_TIER_LOW || tier > MXQ_TIER_HIGH) return MXQ_ERR_MODE;
  if (n_experts <= 0 || n_blocks <= 0) return MXQ_ERR_SHAPE;
  if (sums_off == nullptr || sums_on == nullptr || modes == nullptr) return MXQ_ERR_NULL;
  const double floor_db = kTiers[tier][0], w4a8_db = kTiers[tier][1], margin = kTiers[tier][2];
  const size_t n = (size_t)n_experts * (size_t)n_blocks;
  for (size_t i = 0; i < n; ++i) {
    const double off = sqnr_of(sums_off + 2 * i), on = sqnr_of(sums_on + 2 * i);
    const double best = off > on ? off : on;
    uint8_t m;
    if (best < floor_db) m = MXQ_POLICY_BF16;
    else if (best < w4a8_db) m = MXQ_W4A8;
    else if (on - off > margin) m = MXQ_POLICY_TRANSFORM_ON;
    else m = MXQ_W4A4;
    modes[i] = m;
  }
  return MXQ_OK;
}

int mxq_fp8_calibrate(const void* x, int64_t M, int64_t K, int64_t ldx, float* amax, hipStream_t stream) {
  int st = check_mk(M, K, ldx);
  if (st != MXQ_OK) return st;
  if (M == 0) return MXQ_OK;
  if (x == nullptr || amax == nullptr) return MXQ_ERR_NULL;
  if (!aligned16(x) || ldx % 8 != 0 || (reinterpret_cast<uintptr_t>(amax) & 3u) != 0) return MXQ_ERR_ALIGN;
  if (log_enabled()) fprintf(stderr, "[mxq] fp8_calibrate M=%lld K=%lld\n", (long long)M, (long long)K);
  if ((st = finite_guard("calibration input", x, M, K, ldx, stream)) != MXQ_OK) return st;
  return hip_status(mxq::launch_fp8_amax(x, M, K, ldx, amax, stream));
}

int mxq_quantize_act_fp8_static(const void* x, int64_t M, int64_t K, int64_t ldx, const float* amax,
                                void* codes, void* scales, hipStream_t stream) {
  int st = check_mk(M, K, ldx);
  if (st != MXQ_OK) return st;
  if (M == 0) return MXQ_OK;
  if (x == nullptr || amax == nullptr || codes == nullptr || scales == nullptr) return MXQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales) || ldx % 8 != 0 ||
      (reinterpret_cast<uintptr_t>(amax) & 3u) != 0)
    return MXQ_ERR_ALIGN;
  if (log_enabled()) fprintf(stderr, "[mxq] quantize_act fp8_static M=%lld K=%lld\n", (long long)M, (long long)K);
  if ((st = finite_guard("activation", x, M, K, ldx, stream)) != MXQ_OK) return st;
  return hip_status(mxq::launch_fp8_static_quant(x, M, K, ldx, amax, codes, scales, stream));
}

int mxq_gemm(int mode, const void* a_codes, const void* a_scales,
             const void* w_codes, const void* w_scales, const void* bias,
             int epilogue, void* y, int64_t M, int64_t N, int64_t K,
             hipStream_t stream) {
  if (mode != MXQ_W4A4 && mode != MXQ_W4A8) return MXQ_ERR_MODE;
  if (epilogue != MXQ_EPI_NONE && epilogue != MXQ_EPI_GELU_TANH) return MXQ_ERR_MODE;
  int st = check_mk(M, K, K);
  if (st != MXQ_OK) return st;
  if (N < 0 || N >= kMaxDim) return MXQ_ERR_SHAPE;
  if (M == 0 || N == 0) return MXQ_OK;
  if (a_codes == nullptr || a_scales == nullptr || w_codes == nullptr || w_scales == nullptr || y == nullptr)
    return MXQ_ERR_NULL;
  if (!aligned16(a_codes) || !aligned16(a_scales) || !aligned16(w_codes) || !aligned16(w_scales) ||
      !aligned16(y) || (bias != nullptr && !aligned16(bias)))
    return MXQ_ERR_ALIGN;
  if (log_enabled())
    fprintf(stderr, "[mxq] gemm %s M=%lld N=%lld K=%lld epi=%d kernel=%s\n", mode == MXQ_W4A4 ? "w4a4" : "w4a8",
            (long long)M, (long long)N, (long long)K, epilogue, mxq::gemm_variant_name(mode, M, N, K));
  return output_guard(mxq::launch_gemm(mode, a_codes, a_scales, w_codes, w_scales, bias, epilogue, y, M, N, K, stream),
                      "output", y, M, N, stream);
}

int mxq_gemm_mxfp4_out(const void* a_codes, const void* a_scales, const void* w_codes, const void* w_scales,
                       const void* bias, int epilogue, void* y_codes, void* y_scales, int64_t M, int64_t N,
                       int64_t K, hipStream_t stream) {
  if (epilogue != MXQ_EPI_NONE && epilogue != MXQ_EPI_GELU_TANH) return MXQ_ERR_MODE;
  int st = check_mk(M, K, K);
  if (st != MXQ_OK) return st;
  if (N < 0 || N >= kMaxDim) return MXQ_ERR_SHAPE;
  if (M == 0 || N == 0) return MXQ_OK;
  if (!mxq::gemm_mxfp4_out_supported(M, N, K)) return MXQ_ERR_SHAPE;
  if (a_codes == nullptr || a_scales == nullptr || w_codes == nullptr || w_scales == nullptr || y_codes == nullptr ||
      y_scales == nullptr)
    return MXQ_ERR_NULL;
  if (!aligned16(a_codes) || !aligned16(a_scales) || !aligned16(w_codes) || !aligned16(w_scales) ||
      !aligned16(y_codes) || !aligned16(y_scales) || (bias != nullptr && !aligned16(bias)))
    return MXQ_ERR_ALIGN;
  if (log_enabled())
    fprintf(stderr, "[mxq] gemm w4a4 -> mxfp4 M=%lld N=%lld K=%lld epi=%d\n", (long long)M, (long long)N,
            (long long)K, epilogue);
  return hip_status(mxq::launch_gemm_mxfp4_out(a_codes, a_scales, w_codes, w_scales, bias, epilogue, y_codes,
                                               y_scales, M, N, K, stream));
}

int mxq_gemm_mxfp4_hadamard_out(const void* a_codes, const void* a_scales, const void* w_codes, const void* w_scales,
                                const void* bias, int epilogue, const float* mult, void* y_codes, void* y_scales,
                                int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  if (epilogue != MXQ_EPI_NONE && epilogue != MXQ_EPI_GELU_TANH) return MXQ_ERR_MODE;
  int st = check_mk(M, K, K);
  if (st != MXQ_OK) return st;
  if (N < 0 || N >= kMaxDim) return MXQ_ERR_SHAPE;
  if (M == 0 || N == 0) return MXQ_OK;
  if (!mxq::gemm_mxfp4_out_supported(M, N, K)) return MXQ_ERR_SHAPE;
  if (a_codes == nullptr || a_scales == nullptr || w_codes == nullptr || w_scales == nullptr || mult == nullptr ||
      y_codes == nullptr || y_scales == nullptr)
    return MXQ_ERR_NULL;
  if (!aligned16(a_codes) || !aligned16(a_scales) || !aligned16(w_codes) || !aligned16(w_scales) ||
      !aligned16(mult) || !aligned16(y_codes) || !aligned16(y_scales) || (bias != nullptr && !aligned16(bias)))
    return MXQ_ERR_ALIGN;
  if (log_enabled())
    fprintf(stderr, "[mxq] gemm w4a4 -> transformed mxfp4 M=%lld N=%lld K=%lld epi=%d\n", (long long)M,
            (long long)N, (long long)K, epilogue);
  return hip_status(mxq::launch_gemm_mxfp4_hadamard_out(a_codes, a_scales, w_codes, w_scales, bias, epilogue, mult,
                                                        y_codes, y_scales, M, N, K, stream));
}

int mxq_gemm_fp8_static_out(const void* a_codes, const void* a_scales, const void* w_codes, const void* w_scales,
                            const void* bias, int epilogue, const float* out_amax, void* y_codes, void* y_scales,
                            int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  if (epilogue != MXQ_EPI_NONE && epilogue != MXQ_EPI_GELU_TANH) return MXQ_ERR_MODE;
  int st = check_mk(M, K, K);
  if (st != MXQ_OK) return st;
  if (N < 0 || N >= kMaxDim) return MXQ_ERR_SHAPE;
  if (M == 0 || N == 0) return MXQ_OK;
  if (!mxq::gemm_fp8_static_out_supported(M, N, K)) return MXQ_ERR_SHAPE;
  if (a_codes == nullptr || a_scales == nullptr || w_codes == nullptr || w_scales == nullptr ||
      out_amax == nullptr || y_codes == nullptr || y_scales == nullptr)
    return MXQ_ERR_NULL;
  if (!aligned16(a_codes) || !aligned16(a_scales) || !aligned16(w_codes) || !aligned16(w_scales) ||
      !aligned16(y_codes) || !aligned16(y_scales) || (bias != nullptr && !aligned16(bias)) ||
      (reinterpret_cast<uintptr_t>(out_amax) & 3u) != 0)
    return MXQ_ERR_ALIGN;
  if (log_enabled())
    fprintf(stderr, "[mxq] gemm w4a8 -> fp8 static M=%lld N=%lld K=%lld epi=%d\n", (long long)M, (long long)N,
            (long long)K, epilogue);
  return hip_status(mxq::launch_gemm_fp8_static_out(a_codes, a_scales, w_codes, w_scales, bias, epilogue, out_amax,
                                                    y_codes, y_scales, M, N, K, stream));
}

static int mxfp4_layout_call(bool to_canonical, const void* src_codes, const void* src_scales, int64_t rows,
                             int64_t K, void* dst_codes, void* dst_scales, hipStream_t stream) {
  int st = check_mk(rows, K, K);
  if (st != MXQ_OK) return st;
  if (rows == 0) return MXQ_OK;
  if (src_codes == nullptr || src_scales == nullptr || dst_codes == nullptr || dst_scales == nullptr)
    return MXQ_ERR_NULL;
  if (!aligned16(src_codes) || !aligned16(src_scales) || !aligned16(dst_codes) || !aligned16(dst_scales))
    return MXQ_ERR_ALIGN;
  if (log_enabled())
    fprintf(stderr, "[mxq] mxfp4 layout %s rows=%lld K=%lld\n", to_canonical ? "-> canonical" : "<- canonical",
            (long long)rows, (long long)K);
  return hip_status(mxq::launch_mxfp4_layout(to_canonical, src_codes, src_scales, rows, K, dst_codes, dst_scales,
                                             stream));
}

int mxq_mxfp4_to_canonical(const void* codes, const void* scales, int64_t rows, int64_t K, void* codes_rm,
                           void* scales_rm, hipStream_t stream) {
  return mxfp4_layout_call(true, codes, scales, rows, K, codes_rm, scales_rm, stream);
}

int mxq_mxfp4_from_canonical(const void* codes_rm, const void* scales_rm, int64_t rows, int64_t K, void* codes,
                             void* scales, hipStream_t stream) {
  return mxfp4_layout_call(false, codes_rm, scales_rm, rows, K, codes, scales, stream);
}

const char* mxq_gemm_kernel_name(int mode, int64_t M, int64_t N, int64_t K) {
  if (mode != MXQ_W4A4 && mode != MXQ_W4A8) return "invalid";
  return mxq::gemm_variant_name(mode, M, N, K);
}

int mxq_policy_create(const uint8_t* modes, int32_t n_experts, int32_t n_blocks, void** policy) {
  if (policy == nullptr) return MXQ_ERR_NULL;
  *policy = nullptr;
  if (n_experts <= 0 || n_blocks <= 0) return MXQ_ERR_SHAPE;
  if (modes == nullptr) return MXQ_ERR_NULL;
  const size_t n = (size_t)n_experts * (size_t)n_blocks;
  for (size_t i = 0; i < n; ++i)
    if (modes[i] != MXQ_W4A4 && modes[i] != MXQ_W4A8 && modes[i] != MXQ_POLICY_TRANSFORM_ON) {
      if (log_enabled())
        fprintf(stderr, "[mxq] policy_create: expert %lld block %lld has mode %d (not W4A4, W4A8 or transform_on)\n",
                (long long)(i / (size_t)n_blocks), (long long)(i % (size_t)n_blocks), (int)modes[i]);
      return MXQ_ERR_MODE;
    }
  Policy* p = new (std::nothrow) Policy;
  if (p == nullptr) return MXQ_ERR_HIP;
  p->n_experts = n_experts;
  p->n_blocks = n_blocks;
  p->modes.assign(modes, modes + n);
  *policy = p;
  return MXQ_OK;
}

int mxq_policy_destroy(void* policy) {
  delete static_cast<Policy*>(policy);
  return MXQ_OK;
}

int mxq_policy_mode(const void* policy, int32_t expert, int32_t block, int* mode) {
  if (policy == nullptr || mode == nullptr) return MXQ_ERR_NULL;
  const Policy* p = static_cast<const Policy*>(policy);
  if (expert < 0 || expert >= p->n_experts || block < 0 || block >= p->n_blocks) return MXQ_ERR_RANGE;
  *mode = p->modes[(size_t)expert * (size_t)p->n_blocks + (size_t)block];
  return MXQ_OK;
}

int mxq_qlinear_workspace_bytes(int mode, int64_t M, int64_t K, size_t* bytes) {
  if (bytes == nullptr) return MXQ_ERR_NULL;
  if (mode != MXQ_W4A4 && mode != MXQ_W4A8 && mode != MXQ_POLICY_TRANSFORM_ON) return MXQ_ERR_MODE;
  int st = check_mk(M, K, K);
  if (st != MXQ_OK) return st;
  size_t cb = 0;
  workspace_layout(mode == MXQ_W4A8 ? MXQ_W4A8 : MXQ_W4A4, M, K, &cb, bytes);
  return MXQ_OK;
}

// Shared body of mxq_qlinear and mxq_qlinear_transform: `allow_transform`
// says whether a transform_on block may run (with act_mult).
static int qlinear_impl(const void* policy, int32_t expert, int32_t block, const void* x, int64_t M, int64_t K,
                        const void* w_codes, const void* w_scales, int64_t N, const void* bias, int epilogue,
                        bool allow_transform, const float* act_mult, void* y, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  int mode = 0;
  int st = mxq_policy_mode(policy, expert, block, &mode);
  if (st != MXQ_OK) return st;
  const bool transform = mode == MXQ_POLICY_TRANSFORM_ON;
  if (transform && !allow_transform) return MXQ_ERR_MODE;
  if (epilogue != MXQ_EPI_NONE && epilogue != MXQ_EPI_GELU_TANH) return MXQ_ERR_MODE;
  st = check_mk(M, K, K);
  if (st != MXQ_OK) return st;
  if (transform && K % 128 != 0) return MXQ_ERR_SHAPE;
  if (N < 0 || N >= kMaxDim) return MXQ_ERR_SHAPE;
  if (M == 0 || N == 0) return MXQ_OK;
  if (x == nullptr || w_codes == nullptr || w_scales == nullptr || y == nullptr) return MXQ_ERR_NULL;
  if (transform && act_mult == nullptr) return MXQ_ERR_NULL;
  if (workspace == nullptr) return MXQ_ERR_WORKSPACE;
  const int gemm_mode = mode == MXQ_W4A8 ? MXQ_W4A8 : MXQ_W4A4;
  size_t codes_bytes = 0, need = 0;
  workspace_layout(gemm_mode, M, K, &codes_bytes, &need);
  if (workspace_bytes < need) return MXQ_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(w_codes) || !aligned16(w_scales) || !aligned16(y) ||
      !aligned16(workspace) || (bias != nullptr && !aligned16(bias)) || (transform && !aligned16(act_mult)))
    return MXQ_ERR_ALIGN;
  void* a_codes = workspace;
  void* a_scales = static_cast<uint8_t*>(workspace) + codes_bytes;
  st = transform ? mxq_quantize_mxfp4_hadamard(x, M, K, K, act_mult, a_codes, a_scales, stream)
                 : mxq_quantize_act(mode, x, M, K, K, a_codes, a_scales, stream);
  if (st != MXQ_OK) return st;
  return mxq_gemm(gemm_mode, a_codes, a_scales, w_codes, w_scales, bias, epilogue, y, M, N, K, stream);
}

int mxq_qlinear(const void* policy, int32_t expert, int32_t block,
                const void* x, int64_t M, int64_t K,
                const void* w_codes, const void* w_scales, int64_t N,
                const void* bias, int epilogue, void* y,
                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return qlinear_impl(policy, expert, block, x, M, K, w_codes, w_scales, N, bias, epilogue, false, nullptr, y,
                      workspace, workspace_bytes, stream);
}

int mxq_qlinear_transform(const void* policy, int32_t expert, int32_t block,
                          const void* x, int64_t M, int64_t K,
                          const void* w_codes, const void* w_scales, int64_t N,
                          const void* bias, int epilogue, const float* act_mult, void* y,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return qlinear_impl(policy, expert, block, x, M, K, w_codes, w_scales, N, bias, epilogue, true, act_mult, y,
                      workspace, workspace_bytes, stream);
}

}  // extern "C"
