// Default-layout GEMM launches: tile shapes 64 and 128 run gemm_kernel (gemm_kernel.hpp, four
// waves), 256 runs gemm_pp_kernel (gemm_pp_kernel.hpp, eight waves); four input/output type
// combinations each, and the occupancy query. K = 0 runs gemm_zero_kernel instead.
#include "gemm_pp_kernel.hpp"

namespace tbl {
namespace {

typedef unsigned zero16_t __attribute__((ext_vector_type(4)));
constexpr int kZeroThreads = 256;
constexpr int64_t kMaxZeroBlocks = int64_t{1} << 20;

// K = 0: every element of C is an empty sum, +0, whose bits are all zero in fp16, bf16 and fp32.
// 16 bytes per lane over a grid-stride loop; the last bytes (C holds 2- or 4-byte elements, so
// fewer than 16 and an even count) are written two at a time by the first lane.
__global__ __launch_bounds__(kZeroThreads) void gemm_zero_kernel(unsigned char* __restrict__ c, int64_t bytes) {
  const int64_t chunks = bytes / 16;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kZeroThreads;
  zero16_t* c16 = reinterpret_cast<zero16_t*>(c);
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kZeroThreads + threadIdx.x; i < chunks; i += stride)
    c16[i] = zero16_t{0u, 0u, 0u, 0u};
  if (blockIdx.x == 0 && threadIdx.x == 0)
    for (int64_t b = chunks * 16; b + 2 <= bytes; b += 2) *reinterpret_cast<uint16_t*>(c + b) = 0;
}

}  // namespace

hipError_t launch_gemm_zero(void* C, int64_t bytes, hipStream_t s) {
  const int64_t want = (bytes / 16 + kZeroThreads - 1) / kZeroThreads;
  const int64_t blocks = want < 1 ? 1 : want < kMaxZeroBlocks ? want : kMaxZeroBlocks;
  hipLaunchKernelGGL(gemm_zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kZeroThreads), 0, s,
                     static_cast<unsigned char*>(C), bytes);
  return hipGetLastError();
}

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
