// int32 matrix transpose staged through a 64 x 64 LDS tile, in three LDS layouts.
//
// Follows "CUDA Swizzle & bank conflict" (whc-imageprocess.github.io), section
// "Case Study / Matrix Transpose": a workgroup reads its input tile row by row (coalesced), stores
// every element into shared memory at the transposed logical position [col][row], and after a
// barrier reads shared memory row by row and writes the output tile row by row (coalesced). The
// transposed store is what conflicts: the lanes of one wave write one logical column. The three
// layouts are the page's naive, padded (+1 element per row) and XOR (physical column = column XOR
// row) layouts, sized here to a 64 x 64 tile and 64-lane waves.
//
// Workgroup: 64 x 4 threads; thread (x, y) handles rows y, y+4, ..., y+60 of the tile, so each
// wave covers one full tile row per instruction. The barrier is unconditional (sizes are tile
// multiples), unlike the page's kernels where it sits inside a bounds check.
#include <stdint.h>

#include "internal.hpp"

namespace tbl {
namespace {

constexpr int kTile = 64;
constexpr int kRowsPerPass = 4;

template <int kLayout>
__device__ __forceinline__ int lds_index(int r, int c) {
  if constexpr (kLayout == 0) return r * kTile + c;          // naive
  else if constexpr (kLayout == 1) return r * (kTile + 1) + c;  // padded
  else return r * kTile + (c ^ r);                            // XOR
}

template <int kLayout>
__global__ __launch_bounds__(kTile * kRowsPerPass) void transpose_kernel(
    const int32_t* __restrict__ in, int32_t* __restrict__ out, int rows, int cols) {
  __shared__ int32_t tile[kTile * (kTile + 1)];
  const int x = threadIdx.x, y = threadIdx.y;
  const size_t r0 = static_cast<size_t>(blockIdx.y) * kTile;
  const size_t c0 = static_cast<size_t>(blockIdx.x) * kTile;

  int32_t v[kTile / kRowsPerPass];
#pragma unroll
  for (int i = 0; i < kTile / kRowsPerPass; ++i) {
    const int r = y + kRowsPerPass * i;
    v[i] = in[(r0 + r) * cols + c0 + x];
  }
#pragma unroll
  for (int i = 0; i < kTile / kRowsPerPass; ++i) {
    const int r = y + kRowsPerPass * i;
    tile[lds_index<kLayout>(x, r)] = v[i];     // element (r, x) of the input tile at [x][r]
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kTile / kRowsPerPass; ++i) {
    const int r = y + kRowsPerPass * i;
    out[(c0 + r) * rows + r0 + x] = tile[lds_index<kLayout>(r, x)];
  }
}

}  // namespace

hipError_t launch_transpose_i32(const int32_t* in, int32_t* out, int rows, int cols, int layout,
                                hipStream_t s) {
  const dim3 grid(cols / kTile, rows / kTile), block(kTile, kRowsPerPass);
  switch (layout) {
    case 0: hipLaunchKernelGGL(transpose_kernel<0>, grid, block, 0, s, in, out, rows, cols); break;
    case 1: hipLaunchKernelGGL(transpose_kernel<1>, grid, block, 0, s, in, out, rows, cols); break;
    case 2: hipLaunchKernelGGL(transpose_kernel<2>, grid, block, 0, s, in, out, rows, cols); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tbl
