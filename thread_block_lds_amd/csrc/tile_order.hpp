// Tile orders: tile id t -> output tile (m, n), evaluated on the device by the GEMM's tile loop and
// by the tile_map kernel (one definition for both, so the dumped table is the executed schedule).
//
// Orders follow "CUDA Thread Block Swizzle" (leimao.github.io): sections "Linear Swizzle",
// "Grouped 2D Panel Swizzle", "Morton / Z-order Swizzle", "Bitwise XOR Swizzle" and the pid-mapping
// functions of its benchmark script; group-major and serpentine follow the tvm_tirx
// ClusterPersistentScheduler2D page ("Tile Ordering", "Serpentine Mode"). The serpentine order is
// the column-strip reading that reproduces that page's 4x4 table. The two-level (cluster) form
// follows that page's "Example 2": an order walks a grid of cluster tiles of cm x cn tiles, and the
// cm * cn consecutive ids of one cluster expand its cluster tile by their rank. The XCD remap is this
// library's addition for gfx950's eight private L2s; applied before the cluster split, it places a
// cluster's ids on one XCD.
//
// All quantities are wave-uniform, so in the GEMM they live in scalar registers. Every division is
// by a launch constant whose reciprocal the host computes once (FastDiv), so a division costs a
// scalar multiply-high, a multiply and one correction, and nothing needs hoisting out of loops.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tbl {

enum Order : int { kRow = 0, kCol = 1, kPanel = 2, kMorton = 3, kXor = 4, kSerpentine = 5 };
constexpr int kXcdRemapFlag = 0x100;
constexpr int kNumXcds = 8;

// Division of a 32-bit unsigned n by a fixed d >= 1 through m = floor(2^32 / d) (0 when d = 1):
// q0 = (n * m) >> 32 satisfies floor(n/d) - 1 <= q0 <= floor(n/d), so one correction is exact.
struct FastDiv {
  unsigned d;
  unsigned m;
};

inline FastDiv make_fastdiv(unsigned d) {
  FastDiv f;
  f.d = d;
  f.m = d <= 1 ? 0u : static_cast<unsigned>((uint64_t{1} << 32) / d);
  return f;
}

__host__ __device__ inline unsigned fdiv(unsigned n, FastDiv f) {
  if (f.d == 1) return n;
  unsigned q = static_cast<unsigned>((static_cast<uint64_t>(n) * f.m) >> 32);
  if (n - q * f.d >= f.d) ++q;
  return q;
}

__host__ __device__ inline unsigned fmod_(unsigned n, FastDiv f) { return n - fdiv(n, f) * f.d; }

struct TileOrder {
  int mode;      // kRow .. kSerpentine
  int remap;     // 1: apply the XCD remap before the order
  int grid_m;    // rows of the grid the order walks (cluster tiles when clustered)
  int grid_n;    // its columns
  int group;     // panel group / serpentine strip width, clamped by the host to [1, grid]
  int tiles;     // output tiles: grid_m * grid_n * cluster size
  int cm;        // cluster rows (1: no clusters)
  int cn;        // cluster columns
  FastDiv div_cs;        // cm * cn
  FastDiv div_cm;        // cm
  FastDiv div_m;         // grid_m
  FastDiv div_n;         // grid_n
  FastDiv div_span;      // panel: group * grid_n ids per group; serpentine: group * grid_m per strip
  FastDiv div_full;      // panel: group rows; serpentine: group columns
  FastDiv div_last;      // the same for the last, partial group / strip
};

// Round-robin dispatch puts workgroup w on XCD w % 8. Give XCD d the ids d*(T8/8) .. (d+1)*(T8/8)-1
// of the order, in the order its workgroups arrive; ids past the last full group of 8 stay put.
__host__ __device__ inline int xcd_remap(int t, int tiles) {
  const int t8 = tiles & ~(kNumXcds - 1);
  if (t >= t8) return t;
  return (t & (kNumXcds - 1)) * (t8 / kNumXcds) + (t >> 3);
}

// Gather the even bits of a 32-bit id into the low 16 bits.
__host__ __device__ inline unsigned compact_even_bits(unsigned x) {
  x &= 0x55555555u;
  x = (x | (x >> 1)) & 0x33333333u;
  x = (x | (x >> 2)) & 0x0F0F0F0Fu;
  x = (x | (x >> 4)) & 0x00FF00FFu;
  x = (x | (x >> 8)) & 0x0000FFFFu;
  return x;
}

__host__ __device__ inline void order_tile(const TileOrder& o, int t_in, int& m, int& n) {
  const unsigned tr = static_cast<unsigned>(o.remap ? xcd_remap(t_in, o.tiles) : t_in);
  // cluster id and rank (identity when the cluster is one tile)
  const unsigned t = fdiv(tr, o.div_cs);
  const unsigned rank = tr - t * o.div_cs.d;
  switch (o.mode) {
    case kRow: {
      const unsigned q = fdiv(t, o.div_n);
      m = static_cast<int>(q);
      n = static_cast<int>(t - q * o.div_n.d);
      break;
    }
    case kCol: {
      const unsigned q = fdiv(t, o.div_m);
      n = static_cast<int>(q);
      m = static_cast<int>(t - q * o.div_m.d);
      break;
    }
    case kPanel: {
      // groups of `group` rows; the row inside a group is t modulo the group's height
      const unsigned grp = fdiv(t, o.div_span);
      const unsigned first = grp * o.div_full.d;
      const unsigned in_group = t - grp * o.div_span.d;
      const bool last = first + o.div_full.d > static_cast<unsigned>(o.grid_m);
      const FastDiv h = last ? o.div_last : o.div_full;
      m = static_cast<int>(first + fmod_(t, h));
      n = static_cast<int>(fdiv(in_group, h));
      break;
    }
    case kMorton:
      m = static_cast<int>(fmod_(compact_even_bits(t), o.div_m));
      n = static_cast<int>(fmod_(compact_even_bits(t >> 1), o.div_n));
      break;
    case kXor: {
      const unsigned y = fdiv(t, o.div_n);
      const unsigned x = t - y * o.div_n.d;
      m = static_cast<int>(fmod_(x ^ y, o.div_m));
      n = static_cast<int>(fmod_(y, o.div_n));
      break;
    }
    default: {  // kSerpentine: column strips of `group` columns, alternate strips walked upwards
      const unsigned k = fdiv(t, o.div_span);
      const unsigned u = t - k * o.div_span.d;
      const bool last = (k + 1) * o.div_full.d > static_cast<unsigned>(o.grid_n);
      const FastDiv w = last ? o.div_last : o.div_full;
      const unsigned r = fdiv(u, w);
      m = static_cast<int>((k & 1) ? static_cast<unsigned>(o.grid_m) - 1 - r : r);
      n = static_cast<int>(k * o.div_full.d + (u - r * w.d));
      break;
    }
  }
  if (o.div_cs.d > 1) {
    const unsigned cb_n = fdiv(rank, o.div_cm);
    m = m * o.cm + static_cast<int>(rank - cb_n * o.div_cm.d);
    n = n * o.cn + static_cast<int>(cb_n);
  }
}

// Host: the complete order description for a launch. gm x gn is the grid the order walks (the
// cluster-tile grid when cm * cn > 1); the group is already clamped to it.
inline TileOrder make_tile_order(int mode, int remap, int gm, int gn, int group, int cm = 1, int cn = 1) {
  TileOrder o;
  o.mode = mode;
  o.remap = remap;
  o.grid_m = gm;
  o.grid_n = gn;
  o.group = group;
  o.tiles = gm * gn * cm * cn;
  o.cm = cm;
  o.cn = cn;
  o.div_cs = make_fastdiv(static_cast<unsigned>(cm * cn));
  o.div_cm = make_fastdiv(static_cast<unsigned>(cm));
  o.div_m = make_fastdiv(static_cast<unsigned>(gm));
  o.div_n = make_fastdiv(static_cast<unsigned>(gn));
  if (mode == kPanel) {
    o.div_span = make_fastdiv(static_cast<unsigned>(group * gn));
    o.div_full = make_fastdiv(static_cast<unsigned>(group));
    const int rem = gm % group;
    o.div_last = make_fastdiv(static_cast<unsigned>(rem == 0 ? group : rem));
  } else if (mode == kSerpentine) {
    o.div_span = make_fastdiv(static_cast<unsigned>(group * gm));
    o.div_full = make_fastdiv(static_cast<unsigned>(group));
    const int rem = gn % group;
    o.div_last = make_fastdiv(static_cast<unsigned>(rem == 0 ? group : rem));
  } else {
    o.div_span = o.div_full = o.div_last = make_fastdiv(1);
  }
  return o;
}

}  // namespace tbl
