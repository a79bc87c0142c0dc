// Sustained matrix-pipe rate on given operand data: the GEMM's inner MFMA stream without its memory
// traffic.
//
// Every wave loads four 16-byte A fragments and four B fragments from the caller's operands once,
// then issues `iters` rounds of 32 independent v_mfma_f32_16x16x32_{f16,bf16} accumulations in the
// order the GEMM's wave issues them: the A fragment (second operand) changes every fourth MFMA, and
// the B fragments (first operand) run forward and backward in turn, so B stays where A changes. Nothing else runs in the loop, so the rate this kernel
// reaches is what the matrix pipes sustain at the core clock the chip holds for this data: the
// clock, and with it the rate, falls as the operands' switching activity (and power) rises. The
// register budget is the GEMM's (512 threads per workgroup allowed, so at most 256 registers per
// lane), which keeps the accumulators in VGPRs as they are in the GEMM.
#include <stdint.h>

#include "internal.hpp"

namespace tbl {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <bool kBf16>
__device__ __forceinline__ f32x4_t mfma(uint4 a, uint4 b, f32x4_t c) {
  if constexpr (kBf16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                  __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
  }
}

template <bool kBf16>
__global__ __launch_bounds__(512) void mfma_rate_kernel(const uint4* __restrict__ A,
                                                        const uint4* __restrict__ B, int64_t chunks,
                                                        int iters, float* __restrict__ out,
                                                        int64_t* __restrict__ cycles) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  uint4 a[4], b[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t c = ((wave * 4 + q) * 64 + lane) % chunks;   // 8 consecutive 16-bit values
    a[q] = A[c];
    b[q] = B[c];
  }
  f32x4_t acc[32];
#pragma unroll
  for (int j = 0; j < 32; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[j][r] = 0.f;
  __syncthreads();
  const uint64_t clk0 = __builtin_readcyclecounter();
  const uint64_t rt0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int q = 0; q < 32; ++q) acc[q] = mfma<kBf16>(b[((q >> 2) & 1) ? 3 - (q & 3) : (q & 3)], a[(q >> 2) & 3], acc[q]);
  }
  const uint64_t clk1 = __builtin_readcyclecounter();
  const uint64_t rt1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 32; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) s += acc[j][r];
  out[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = s;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    cycles[0] = static_cast<int64_t>(clk1 - clk0);
    cycles[1] = static_cast<int64_t>(rt1 - rt0);
  }
}

}  // namespace

hipError_t launch_mfma_rate(const void* A, const void* B, int64_t elems, bool bf16, int workgroups,
                            int iters, float* out, int64_t* cycles, hipStream_t s) {
  const int64_t chunks = elems / 8;
  if (bf16) {
    hipLaunchKernelGGL(mfma_rate_kernel<true>, dim3(workgroups), dim3(256), 0, s,
                       static_cast<const uint4*>(A), static_cast<const uint4*>(B), chunks, iters, out,
                       cycles);
  } else {
    hipLaunchKernelGGL(mfma_rate_kernel<false>, dim3(workgroups), dim3(256), 0, s,
                       static_cast<const uint4*>(A), static_cast<const uint4*>(B), chunks, iters, out,
                       cycles);
  }
  return hipGetLastError();
}

}  // namespace tbl
