// Tile orders: tile id t -> output tile (m, n), evaluated on the device by the GEMM's tile loop and
// by the tile_map kernel (one definition for both, so the dumped table is the executed schedule).
//
// Orders follow "CUDA Thread Block Swizzle" (leimao.github.io): sections "Linear Swizzle",
// "Grouped 2D Panel Swizzle", "Morton / Z-order Swizzle", "Bitwise XOR Swizzle" and the pid-mapping
// functions of its benchmark script; group-major and serpentine follow the tvm_tirx
// ClusterPersistentScheduler2D page ("Tile Ordering", "Serpentine Mode"). The serpentine order is
// the column-strip reading that reproduces that page's 4x4 table. The XCD remap is this library's
// addition for gfx950's eight private L2s.
//
// All quantities are wave-uniform, so the compiler keeps them in scalar registers.
#pragma once

#include <hip/hip_runtime.h>

namespace tbl {

enum Order : int { kRow = 0, kCol = 1, kPanel = 2, kMorton = 3, kXor = 4, kSerpentine = 5 };
constexpr int kXcdRemapFlag = 0x100;
constexpr int kNumXcds = 8;

struct TileOrder {
  int mode;      // kRow .. kSerpentine
  int remap;     // 1: apply the XCD remap before the order
  int grid_m;    // tile rows
  int grid_n;    // tile columns
  int group;     // panel group / serpentine strip width, already clamped to [1, grid] by the host
  int tiles;     // grid_m * grid_n
};

// Round-robin dispatch puts workgroup w on XCD w % 8. Give XCD d the ids d*(T8/8) .. (d+1)*(T8/8)-1
// of the order, in the order its workgroups arrive; ids past the last full group of 8 stay put.
__host__ __device__ inline int xcd_remap(int t, int tiles) {
  const int t8 = (tiles / kNumXcds) * kNumXcds;
  if (t >= t8) return t;
  return (t % kNumXcds) * (t8 / kNumXcds) + t / kNumXcds;
}

// Gather the even (or odd) bits of a 32-bit id into the low 16 bits.
__host__ __device__ inline unsigned compact_even_bits(unsigned x) {
  x &= 0x55555555u;
  x = (x | (x >> 1)) & 0x33333333u;
  x = (x | (x >> 2)) & 0x0F0F0F0Fu;
  x = (x | (x >> 4)) & 0x00FF00FFu;
  x = (x | (x >> 8)) & 0x0000FFFFu;
  return x;
}

__host__ __device__ inline void order_tile(const TileOrder& o, int t, int& m, int& n) {
  if (o.remap) t = xcd_remap(t, o.tiles);
  const int gm = o.grid_m, gn = o.grid_n;
  switch (o.mode) {
    case kRow:
      m = t / gn;
      n = t % gn;
      break;
    case kCol:
      m = t % gm;
      n = t / gm;
      break;
    case kPanel: {
      const int per_group = o.group * gn;
      const int first = (t / per_group) * o.group;
      const int height = min(gm - first, o.group);
      m = first + t % height;
      n = (t % per_group) / height;
      break;
    }
    case kMorton: {
      const unsigned u = static_cast<unsigned>(t);
      m = static_cast<int>(compact_even_bits(u) % static_cast<unsigned>(gm));
      n = static_cast<int>(compact_even_bits(u >> 1) % static_cast<unsigned>(gn));
      break;
    }
    case kXor: {
      const int x = t % gn, y = t / gn;
      m = (x ^ y) % gm;
      n = y % gn;
      break;
    }
    default: {  // kSerpentine
      const int per_strip = o.group * gm;
      const int k = t / per_strip;
      const int width = min(o.group, gn - k * o.group);
      const int u = t - k * per_strip;
      const int r = u / width;
      m = (k & 1) ? gm - 1 - r : r;
      n = k * o.group + u % width;
      break;
    }
  }
}

}  // namespace tbl
