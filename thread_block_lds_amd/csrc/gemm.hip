// Default-layout GEMM launches: tile shapes 64 and 128 run gemm_kernel (gemm_kernel.hpp, four
// waves), 256 runs gemm_pp_kernel (gemm_pp_kernel.hpp, eight waves); four input/output type
// combinations each, and the occupancy query.
#include "gemm_pp_kernel.hpp"

namespace tbl {
bool gemm_tile_supported(int bm, int bn, int bk) {
  return bk == kBK && bm == bn && (bm == 64 || bm == 128 || bm == 256);
}

hipError_t launch_gemm(int dtype, int bm, int bn, int bk, const GemmLaunch& a, hipStream_t s) {
  if (!gemm_tile_supported(bm, bn, bk)) return hipErrorInvalidValue;
  if (bm == 64) return launch<64, 64>(dtype, a, s);
  if (bm == 128) return launch<128, 128>(dtype, a, s);
  return launch_pp(dtype, a, s);
}

hipError_t launch_gemm_dynamic(int dtype, const GemmLaunch& a, hipStream_t s) {
  return launch_pp_dynamic(dtype, a, s);
}

hipError_t gemm_blocks_per_cu(int dtype, int bm, int bn, int bk, int* out) {
  if (!gemm_tile_supported(bm, bn, bk)) return hipErrorInvalidValue;
  const void* k = bm == 64 ? kernel_for<64, 64>(dtype)
                : bm == 128 ? kernel_for<128, 128>(dtype) : pp_kernel_for(dtype);
  if (k == nullptr) return hipErrorInvalidValue;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(out, k, bm == 256 ? kPPThreads : kThreads, 0);
}

}  // namespace tbl
