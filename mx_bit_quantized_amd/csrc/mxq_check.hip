// mxq_check.hip - the optional non-finite guard (MXQ_CHECK_FINITE). The page
// "Wan q8 performance investigation" records quantized runs that produced
// near-black and all-black frames and calls for guards that fail closed
// instead of passing invalid values on. With MXQ_CHECK_FINITE set, the entry
// points scan their bf16 inputs before enqueueing any work and their bf16
// outputs after it, and return MXQ_ERR_NONFINITE when a value is infinite or
// NaN. A scan synchronizes the stream, so this is a debugging aid, not a
// mode for graph capture or production.
//
// The result goes to `nonfinite_flag`, a static device word of the library on
// each device (its device address from hipGetSymbolAddress, once per device):
// a fill kernel clears it, the scan kernel ORs into it, and the host reads it
// back after the stream has drained. A mutex serializes scans per process.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <mutex>

#include "mxq_internal.h"

namespace {

static __device__ __align__(16) uint32_t nonfinite_flag;

constexpr int kMaxDevices = 64;
std::mutex g_check_mu;
uint32_t* g_flag[kMaxDevices];

}  // namespace

namespace mxq {

constexpr int kScanThreads = 256;

__global__ void flag_clear_kernel(uint32_t* flag) { *flag = 0u; }

// A bf16 value is non-finite when its exponent field is all ones. VEC: each
// thread tests 8 elements per 16-byte load (x 16-byte aligned, ld and cols
// multiples of 8); otherwise one element per load. Rows are looped.
template <bool VEC>
__global__ __launch_bounds__(kScanThreads) void nonfinite_scan_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                                      int64_t cols, int64_t ld,
                                                                      uint32_t* __restrict__ flag) {
  const int64_t per_row = VEC ? cols >> 3 : cols;
  const int64_t n = rows * per_row;
  const int64_t stride = (int64_t)gridDim.x * kScanThreads;
  uint32_t bad = 0;
  for (int64_t t = (int64_t)blockIdx.x * kScanThreads + threadIdx.x; t < n; t += stride) {
    const int64_t r = t / per_row, c = t - r * per_row;
    if constexpr (VEC) {
      const uint4 v = *reinterpret_cast<const uint4*>(x + r * ld + 8 * c);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bad |= (w[i] & 0x7F80u) == 0x7F80u;
        bad |= (w[i] & 0x7F800000u) == 0x7F800000u;
      }
    } else {
      bad |= (x[r * ld + c] & 0x7F80u) == 0x7F80u;
    }
  }
  if (bad) atomicOr(flag, 1u);
}

bool check_finite_enabled() {
  const char* v = getenv("MXQ_CHECK_FINITE");
  return v != nullptr && v[0] != '\0' && v[0] != '0';
}

int scan_nonfinite_bf16(const void* x, int64_t rows, int64_t cols, int64_t ld, hipStream_t s, bool* found) {
  *found = false;
  if (rows <= 0 || cols <= 0) return 0;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 1;
  std::lock_guard<std::mutex> lock(g_check_mu);
  if (g_flag[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(nonfinite_flag)) != hipSuccess || p == nullptr) return 1;
    g_flag[dev] = static_cast<uint32_t*>(p);
  }
  uint32_t* flag = g_flag[dev];
  hipLaunchKernelGGL(flag_clear_kernel, dim3(1), dim3(1), 0, s, flag);
  const bool vec = (reinterpret_cast<uintptr_t>(x) & 15u) == 0 && ld % 8 == 0 && cols % 8 == 0;
  int64_t blocks = (rows * (vec ? cols >> 3 : cols) + kScanThreads - 1) / kScanThreads;
  if (blocks > 4096) blocks = 4096;
  if (vec)
    hipLaunchKernelGGL(nonfinite_scan_kernel<true>, dim3((unsigned)blocks), dim3(kScanThreads), 0, s,
                       static_cast<const uint16_t*>(x), rows, cols, ld, flag);
  else
    hipLaunchKernelGGL(nonfinite_scan_kernel<false>, dim3((unsigned)blocks), dim3(kScanThreads), 0, s,
                       static_cast<const uint16_t*>(x), rows, cols, ld, flag);
  if (hipGetLastError() != hipSuccess) return 1;
  uint32_t host = 0;
  if (hipMemcpyAsync(&host, flag, sizeof(host), hipMemcpyDeviceToHost, s) != hipSuccess) return 1;
  if (hipStreamSynchronize(s) != hipSuccess) return 1;
  *found = host != 0;
  return 0;
}

}  // namespace mxq
