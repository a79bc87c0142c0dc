// tile_map: the forward table t -> (m, n) of a tile order, one lane per tile id, computed with the
// same order_tile() the GEMM's tile loop calls.
#include <stdint.h>

#include "internal.hpp"

namespace tbl {
namespace {

__global__ __launch_bounds__(256) void tile_map_kernel(TileOrder o, int32_t* __restrict__ tile_m,
                                                       int32_t* __restrict__ tile_n) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t < o.tiles) {
    int m, n;
    order_tile(o, t, m, n);
    tile_m[t] = m;
    tile_n[t] = n;
  }
}

}  // namespace

hipError_t launch_tile_map(const TileOrder& o, int32_t* tile_m, int32_t* tile_n, hipStream_t s) {
  const int blocks = (o.tiles + 255) / 256;
  hipLaunchKernelGGL(tile_map_kernel, dim3(blocks), dim3(256), 0, s, o, tile_m, tile_n);
  return hipGetLastError();
}

}  // namespace tbl
