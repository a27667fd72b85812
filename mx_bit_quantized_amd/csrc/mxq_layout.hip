// mxq_layout.hip - conversion between the library's MXFP4 layouts and the
// canonical row-major layout of the OCP MXFP4 format (section "Quantization
// formats" of the page "Quark Mixed-Precision Quantization for Wan2.2 Video
// Generation on AMD Instinct GPUs": OCP MXFP4, its reference [7]).
//
// Canonical: codes [rows][K/2] bytes (element 2t of a row in the low nibble of
// byte t), E8M0 scales [rows][K/32] bytes.
// Library: codes in K panels of 128 elements (panel p holds every row's codes
// of its range, row after row; a ragged last panel is narrower) and scales
// group-major [ceil(K/128)][rows][4], bytes of blocks past K/32 zero.
//
// One MX block (32 elements) is 16 contiguous code bytes in both layouts, so
// each thread moves one block: its 16 code bytes and its scale byte. Threads
// are ordered row-major over (row, block), which makes the row-major side
// contiguous and the panel side runs of 64 bytes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq_internal.h"

namespace mxq {

constexpr int kLayoutThreads = 256;

// byte offset of block j (16 code bytes) of row r in the panel layout
__device__ __forceinline__ int64_t panel_block_offset(int64_t r, int64_t j, int64_t rows, int64_t K) {
  const int64_t p = j >> 2, q = j & 3;
  const int64_t w = K - 128 * p < 128 ? K - 128 * p : 128;  // elements in panel p
  return 64 * p * rows + r * (w >> 1) + 16 * q;
}

// TO_CANONICAL: library -> canonical; otherwise canonical -> library. The
// blocks of a row run over j < KBp = 4 ceil(KB / 4): the library's padding
// scale bytes (j >= KB) are written as zero and never read.
template <bool TO_CANONICAL>
__global__ __launch_bounds__(kLayoutThreads) void mxfp4_layout_kernel(const uint8_t* __restrict__ src_codes,
                                                                      const uint8_t* __restrict__ src_scales,
                                                                      int64_t rows, int64_t K,
                                                                      uint8_t* __restrict__ dst_codes,
                                                                      uint8_t* __restrict__ dst_scales) {
  const int64_t KB = K >> 5, KBp = (KB + 3) & ~int64_t(3);
  const int64_t n = rows * KBp;
  const int64_t stride = (int64_t)gridDim.x * kLayoutThreads;
  for (int64_t t = (int64_t)blockIdx.x * kLayoutThreads + threadIdx.x; t < n; t += stride) {
    const int64_t r = t / KBp, j = t - r * KBp;
    const int64_t gm = ((j >> 2) * rows + r) * 4 + (j & 3);  // group-major scale byte
    if (j < KB) {
      const int64_t pb = panel_block_offset(r, j, rows, K);
      const int64_t rb = r * (K >> 1) + 16 * j;
      if constexpr (TO_CANONICAL) {
        *reinterpret_cast<uint4*>(dst_codes + rb) = *reinterpret_cast<const uint4*>(src_codes + pb);
        dst_scales[r * KB + j] = src_scales[gm];
      } else {
        *reinterpret_cast<uint4*>(dst_codes + pb) = *reinterpret_cast<const uint4*>(src_codes + rb);
        dst_scales[gm] = src_scales[r * KB + j];
      }
    } else if constexpr (!TO_CANONICAL) {
      dst_scales[gm] = 0;
    }
  }
}

hipError_t launch_mxfp4_layout(bool to_canonical, const void* src_codes, const void* src_scales, int64_t rows,
                               int64_t K, void* dst_codes, void* dst_scales, hipStream_t s) {
  const int64_t n = rows * (((K >> 5) + 3) & ~int64_t(3));
  int64_t blocks = (n + kLayoutThreads - 1) / kLayoutThreads;
  if (blocks > 8192) blocks = 8192;  // threads loop beyond
  auto* sc = static_cast<const uint8_t*>(src_codes);
  auto* ss = static_cast<const uint8_t*>(src_scales);
  auto* dc = static_cast<uint8_t*>(dst_codes);
  auto* ds = static_cast<uint8_t*>(dst_scales);
  if (to_canonical)
    hipLaunchKernelGGL(mxfp4_layout_kernel<true>, dim3((unsigned)blocks), dim3(kLayoutThreads), 0, s, sc, ss, rows,
                       K, dc, ds);
  else
    hipLaunchKernelGGL(mxfp4_layout_kernel<false>, dim3((unsigned)blocks), dim3(kLayoutThreads), 0, s, sc, ss, rows,
                       K, dc, ds);
  return hipGetLastError();
}

}  // namespace mxq
