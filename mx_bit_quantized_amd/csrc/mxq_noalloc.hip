// mxq_noalloc.hip - mxq_qlinear without a workspace argument, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc). The activation codes and scales
// that mxq_qlinear writes into the caller's workspace go into `scratch`, a
// fixed array that the library holds on every device it runs on until the
// process ends. Nothing here allocates: the array is part of the code object.
//
// In host code `scratch` names a host-side stand-in, not the device array: its
// device address on the current device comes from hipGetSymbolAddress (once
// per device, kept in g_scratch), and only that address is handed to kernels.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <mutex>

#include "mxq.h"

namespace {

constexpr size_t kScratchBytes = (size_t)MXQ_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch`, per device

// Device address of the current device's scratch array (looked up on the
// first call on that device).
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MXQ_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MXQ_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MXQ_OK;
}

bool log_on() {
  const char* v = getenv("MXQ_LOG");
  return v != nullptr && v[0] != '\0' && v[0] != '0';
}

}  // namespace

extern "C" int mxq_qlinear_noalloc(const void* policy, int32_t expert, int32_t block, const void* x, int64_t M,
                                   int64_t K, const void* w_codes, const void* w_scales, int64_t N, const void* bias,
                                   int epilogue, void* y, hipStream_t stream) {
  int mode = 0;
  int st = mxq_policy_mode(policy, expert, block, &mode);
  if (st != MXQ_OK) return st;
  if (mode != MXQ_W4A4 && mode != MXQ_W4A8) return MXQ_ERR_MODE;  // as mxq_qlinear
  size_t need = 0;
  st = mxq_qlinear_workspace_bytes(mode, M, K, &need);
  if (st != MXQ_OK) return st;
  if (need > kScratchBytes) {
    if (log_on())
      fprintf(stderr, "[mxq] qlinear_noalloc: M=%lld K=%lld needs %zu scratch bytes, more than the %zu it has\n",
              (long long)M, (long long)K, need, kScratchBytes);
    return MXQ_ERR_SCRATCH;
  }
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != MXQ_OK) return st;
  return mxq_qlinear(policy, expert, block, x, M, K, w_codes, w_scales, N, bias, epilogue, y, ws, kScratchBytes,
                     stream);
}
