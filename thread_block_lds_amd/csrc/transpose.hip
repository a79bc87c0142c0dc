// int32 matrix transpose staged through 64 x 64 LDS tiles, in three LDS layouts.
//
// Follows "CUDA Swizzle & bank conflict" (whc-imageprocess.github.io), section
// "Case Study / Matrix Transpose": a tile is read from global memory row by row (coalesced), every
// element is stored into shared memory at the transposed logical position [col][row], and the
// tile is then read from shared memory row by row and written out row by row (coalesced). The
// transposed store is what conflicts: the lanes of one instruction write one logical column. The
// three layouts are the page's naive, padded (+1 element per row) and XOR (physical column =
// column XOR row) layouts, sized here to a 64 x 64 tile and 64-lane waves.
//
// Work split for gfx950: a workgroup of four waves takes a 64-row x 256-column strip of the input,
// and wave w owns the strip's 64 x 64 tile w (columns 64w .. 64w + 63) and its own LDS tile. Each
// load instruction of wave w reads 256 bytes of one input row, and the four waves together read
// 1 KB contiguous per row from one compute unit; each store instruction writes 256 bytes of one
// output row. Per LDS instruction the access pattern is the page's: the transposed store writes
// one logical column (64 lanes, one element each) and the read takes one logical row. Since a
// wave only reads the tile it wrote, a wave-level fence replaces the page's workgroup barrier.
// A last strip narrower than 256 columns (cols a multiple of 64) leaves the idle waves with no work.
#include <stdint.h>

#include "internal.hpp"

namespace tbl {
namespace {

constexpr int kTile = 64;
constexpr int kWaves = 4;                     // tiles per strip
constexpr int kStripCols = kTile * kWaves;    // 256
constexpr int kTileWords = kTile * (kTile + 1);  // room for the padded layout

typedef __attribute__((address_space(3))) int32_t lds_i32_t;

// One 4-byte LDS store per lane, as inline assembly so that the compiler cannot merge a lane's
// consecutive transposed stores (adjacent words in the naive and padded layouts) into wider ones:
// every layout then runs the page's instruction stream, one logical column per store. The memory
// clobber keeps the later LDS reads after the stores.
__device__ __forceinline__ void lds_store_b32(int32_t* p, int32_t v) {
  const unsigned addr = static_cast<unsigned>(reinterpret_cast<uintptr_t>((lds_i32_t*)p));
  asm volatile("ds_write_b32 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

template <int kLayout>
__device__ __forceinline__ int lds_index(int r, int c) {
  if constexpr (kLayout == 0) return r * kTile + c;             // naive
  else if constexpr (kLayout == 1) return r * (kTile + 1) + c;  // padded
  else return r * kTile + (c ^ r);                              // XOR
}

template <int kLayout>
__global__ __launch_bounds__(kTile * kWaves) void transpose_kernel(
    const int32_t* __restrict__ in, int32_t* __restrict__ out, int rows, int cols) {
  __shared__ int32_t lds[kWaves * kTileWords];
  const int lane = threadIdx.x & (kTile - 1);
  const int w = threadIdx.x >> 6;
  const size_t r0 = static_cast<size_t>(blockIdx.y) * kTile;
  const size_t c0 = static_cast<size_t>(blockIdx.x) * kStripCols + static_cast<size_t>(w) * kTile;
  if (c0 >= static_cast<size_t>(cols)) return;   // wave-uniform: this wave's tile is past the edge
  int32_t* tile = lds + w * kTileWords;

  int32_t v[kTile];
#pragma unroll
  for (int e = 0; e < kTile; ++e) v[e] = in[(r0 + e) * cols + c0 + lane];
#pragma unroll
  for (int e = 0; e < kTile; ++e) lds_store_b32(tile + lds_index<kLayout>(lane, e), v[e]);  // (e, lane) at [lane][e]
  // The wave reads only what it wrote, and a wave's LDS operations execute in order: the reads
  // need no workgroup barrier, only to be issued after the stores (the clobber above).
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int e = 0; e < kTile; ++e) out[(c0 + e) * rows + r0 + lane] = tile[lds_index<kLayout>(e, lane)];
}

}  // namespace

hipError_t launch_transpose_i32(const int32_t* in, int32_t* out, int rows, int cols, int layout,
                                hipStream_t s) {
  const dim3 grid((cols + kStripCols - 1) / kStripCols, rows / kTile), block(kTile * kWaves);
  switch (layout) {
    case 0: hipLaunchKernelGGL(transpose_kernel<0>, grid, block, 0, s, in, out, rows, cols); break;
    case 1: hipLaunchKernelGGL(transpose_kernel<1>, grid, block, 0, s, in, out, rows, cols); break;
    case 2: hipLaunchKernelGGL(transpose_kernel<2>, grid, block, 0, s, in, out, rows, cols); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tbl
