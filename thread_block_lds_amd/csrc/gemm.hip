// Default-layout GEMM launches (the kernel is in gemm_kernel.hpp): tile shapes 64, 128 and 256,
// four input/output type combinations, and the occupancy query.
#include "gemm_kernel.hpp"

namespace tbl {
bool gemm_tile_supported(int bm, int bn, int bk) {
  return bk == kBK && bm == bn && (bm == 64 || bm == 128 || bm == 256);
}

hipError_t launch_gemm(int dtype, int bm, int bn, int bk, const GemmLaunch& a, hipStream_t s) {
  if (!gemm_tile_supported(bm, bn, bk)) return hipErrorInvalidValue;
  if (bm == 64) return launch<64, 64>(dtype, a, s);
  if (bm == 128) return launch<128, 128>(dtype, a, s);
  return launch<256, 256>(dtype, a, s);
}

hipError_t gemm_blocks_per_cu(int dtype, int bm, int bn, int bk, int* out) {
  if (!gemm_tile_supported(bm, bn, bk)) return hipErrorInvalidValue;
  const void* k = bm == 64 ? kernel_for<64, 64>(dtype)
                : bm == 128 ? kernel_for<128, 128>(dtype) : kernel_for<256, 256>(dtype);
  if (k == nullptr) return hipErrorInvalidValue;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(out, k, kThreads, 0);
}

}  // namespace tbl
