// A plain device-to-device copy, 16 bytes per lane, optionally with non-temporal accesses: the rate
// this board's HBM sustains for one read stream and one write stream of the same bytes, which is
// the traffic of the int32 transpose ("CUDA Swizzle & bank conflict", section "Case Study / Matrix
// Transpose": every element read once and written once). A measurement aid for the transpose's
// roofline, not part of the method.
//
// Lane i of the grid copies 16-byte chunk i, then i + (grid size), ...; the grid is one workgroup
// per 256 chunks up to 2^20 workgroups, so up to 4 GiB every lane copies one chunk, the fastest
// form measured on gfx950 (a grid-stride loop with several chunks per lane ran 10-12 % slower).
#include <stdint.h>

#include "internal.hpp"

namespace tbl {
namespace {

typedef int v4i32_t __attribute__((ext_vector_type(4)));
constexpr int kCopyThreads = 256;
constexpr int64_t kMaxCopyBlocks = int64_t{1} << 20;

template <bool kNonTemporal>
__global__ __launch_bounds__(kCopyThreads) void copy16_kernel(const v4i32_t* __restrict__ src,
                                                              v4i32_t* __restrict__ dst, int64_t chunks) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kCopyThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kCopyThreads + threadIdx.x; i < chunks; i += stride) {
    if constexpr (kNonTemporal) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
    else dst[i] = src[i];
  }
}

}  // namespace

hipError_t launch_copy16(const void* src, void* dst, int64_t bytes, bool nontemporal, hipStream_t s) {
  const int64_t chunks = bytes / 16;
  const int64_t want = (chunks + kCopyThreads - 1) / kCopyThreads;
  const dim3 grid(static_cast<unsigned>(want < kMaxCopyBlocks ? want : kMaxCopyBlocks)), block(kCopyThreads);
  const auto* in = static_cast<const v4i32_t*>(src);
  auto* out = static_cast<v4i32_t*>(dst);
  if (nontemporal) hipLaunchKernelGGL(copy16_kernel<true>, grid, block, 0, s, in, out, chunks);
  else hipLaunchKernelGGL(copy16_kernel<false>, grid, block, 0, s, in, out, chunks);
  return hipGetLastError();
}

}  // namespace tbl
