// Offline L2 hit-rate prediction for a tile schedule (host code; no HIP call).
//
// "CUDA Thread Block Swizzle" (leimao.github.io), section "CUDA Thread Block Swizzle Benchmark",
// predicts an order's L2 hit rate by replaying the operand blocks that concurrently running tiles
// read through one byte-capacity LRU cache: tiles run in waves of consecutive tile ids, and within
// a wave, k block by k block, each tile reads its A block (m, k), then its B block (k, n). A miss
// inserts the block and evicts least-recently-used blocks while the cache holds more bytes than
// its capacity and more than one block.
//
// gfx950 has eight XCDs with private L2s and dispatches workgroup p to XCD p mod 8, so this
// generalises the replay: `num_caches` caches, program p on cache p mod num_caches, running tile
// ids p, p + P, p + 2P, ... (the stride schedule of the persistent kernel; one id per program when
// P >= T), `resident` programs of a cache at a time in program order. With one cache, P = T and
// resident = the wave size, this is the page's model exactly. The tile order is the one the GEMM
// executes (order_tile).
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "internal.hpp"

namespace tbl {
namespace {

// An LRU over dense block ids: A block (m, k) is m * grid_k + k, B block (k, n) is
// (grid_m + n) * grid_k + k. Recency is a doubly linked list threaded through two arrays;
// head_ is the least recently used block.
class BlockLru {
 public:
  BlockLru(int64_t ids, int64_t a_ids, int64_t a_bytes, int64_t b_bytes, int64_t capacity)
      : prev_(static_cast<size_t>(ids), kAbsent),
        next_(static_cast<size_t>(ids), kNone),
        a_ids_(a_ids),
        a_bytes_(a_bytes),
        b_bytes_(b_bytes),
        capacity_(capacity) {}

  void access(int64_t id) {
    if (prev_[id] != kAbsent) {
      ++hits;
      unlink(id);
      append(id);
      return;
    }
    ++misses;
    append(id);
    ++held_;
    used_ += bytes(id);
    while (used_ > capacity_ && held_ > 1) {
      const int64_t victim = head_;
      unlink(victim);
      prev_[victim] = kAbsent;
      --held_;
      used_ -= bytes(victim);
    }
  }

  int64_t hits = 0;
  int64_t misses = 0;

 private:
  static constexpr int64_t kAbsent = -2;  // in prev_: the block is not held
  static constexpr int64_t kNone = -1;    // list end

  int64_t bytes(int64_t id) const { return id < a_ids_ ? a_bytes_ : b_bytes_; }

  void unlink(int64_t id) {
    const int64_t p = prev_[id], n = next_[id];
    if (p == kNone) head_ = n; else next_[p] = n;
    if (n == kNone) tail_ = p; else prev_[n] = p;
  }

  void append(int64_t id) {
    prev_[id] = tail_;
    next_[id] = kNone;
    if (tail_ == kNone) head_ = id; else next_[tail_] = id;
    tail_ = id;
  }

  std::vector<int64_t> prev_, next_;
  int64_t a_ids_, a_bytes_, b_bytes_, capacity_;
  int64_t head_ = kNone, tail_ = kNone;
  int64_t held_ = 0, used_ = 0;
};

}  // namespace

void predict_l2(const TileOrder& o, int grid_k, int64_t a_bytes, int64_t b_bytes, int64_t capacity,
                int num_caches, int num_programs, int resident, int64_t* hits, int64_t* accesses) {
  const int64_t T = o.tiles, P = num_programs, gk = grid_k;
  // the output-tile grid (the order may walk a grid of cluster tiles)
  const int64_t a_ids = static_cast<int64_t>(o.grid_m) * o.cm * gk;
  const int64_t ids = a_ids + static_cast<int64_t>(o.grid_n) * o.cn * gk;
  std::vector<int64_t> am, bn;  // per running tile of a group: its A and B block ids at k = 0
  *hits = 0;
  *accesses = 0;
  for (int c = 0; c < num_caches; ++c) {
    BlockLru cache(ids, a_ids, a_bytes, b_bytes, capacity);
    // programs of this cache, in order: c, c + num_caches, ... < P; `resident` of them at a time
    const int64_t count = P > c ? (P - c + num_caches - 1) / num_caches : 0;
    for (int64_t g0 = 0; g0 < count; g0 += resident) {
      const int64_t g1 = g0 + resident < count ? g0 + resident : count;
      for (int64_t it = 0;; ++it) {
        am.clear();
        bn.clear();
        for (int64_t j = g0; j < g1; ++j) {
          const int64_t t = c + j * num_caches + it * P;
          if (t >= T) continue;
          int m = 0, n = 0;
          order_tile(o, static_cast<int>(t), m, n);
          am.push_back(static_cast<int64_t>(m) * gk);
          bn.push_back(a_ids + static_cast<int64_t>(n) * gk);
        }
        if (am.empty()) break;
        for (int64_t k = 0; k < gk; ++k)
          for (size_t i = 0; i < am.size(); ++i) {
            cache.access(am[i] + k);
            cache.access(bn[i] + k);
          }
      }
    }
    *hits += cache.hits;
    *accesses += cache.hits + cache.misses;
  }
}

// ---------------------------------------------------------------------------------------------
// Line-granular replay: the same grouping and read order as predict_l2, counted per cache line
// through set-associative caches indexed by address (the GEMM's loads as the L2 sees them).
//
// Each XCD's cache is a flat array of `sets` x `ways` tags (line number + 1; 0 = empty) beside an
// array of last-use stamps from a per-cache counter; a hit restamps its way, a miss fills the
// empty way or the way with the oldest stamp. Within a set that is least-recently-used order.

namespace {

class SetCache {
 public:
  SetCache(const L2Geometry& g)
      : g_(g), tag_(static_cast<size_t>(g.sets * g.ways), 0), stamp_(tag_.size(), 0) {}

  void read_range(uint64_t first, int64_t count) {
    if (count <= 0) return;
    const uint64_t l0 = first / g_.line_bytes, l1 = (first + count - 1) / g_.line_bytes;
    for (uint64_t l = l0; l <= l1; ++l) read_line(l);
  }

  int64_t hits = 0, accesses = 0;

 private:
  void read_line(uint64_t line) {
    const uint64_t fold =
        g_.fold_width > 0 ? (line >> g_.fold_from) & ((uint64_t{1} << g_.fold_width) - 1) : 0;
    const size_t base = static_cast<size_t>((line ^ fold) % static_cast<uint64_t>(g_.sets)) * g_.ways;
    const uint64_t want = line + 1;
    ++accesses;
    ++now_;
    size_t victim = base;
    for (size_t w = base; w < base + g_.ways; ++w) {
      if (tag_[w] == want) {
        ++hits;
        stamp_[w] = now_;
        return;
      }
      if (stamp_[w] < stamp_[victim]) victim = w;  // empty ways carry stamp 0 and win
    }
    tag_[victim] = want;
    stamp_[victim] = now_;
  }

  L2Geometry g_;
  std::vector<uint64_t> tag_, stamp_;
  uint64_t now_ = 0;
};

}  // namespace

void predict_l2_lines(const TileOrder& o, const GemmReadShape& r, const L2Geometry& g, int num_caches,
                      int64_t num_programs, int resident, int64_t* hits, int64_t* accesses) {
  const int64_t T = o.tiles, P = num_programs;
  const int64_t nk = (r.K + r.bk - 1) / r.bk;
  const uint64_t e = static_cast<uint64_t>(r.elem_bytes);
  struct Tile {
    int64_t row0, row1, col0, col1;
  };
  std::vector<Tile> group;
  *hits = 0;
  *accesses = 0;
  for (int c = 0; c < num_caches; ++c) {
    SetCache cache(g);
    const int64_t count = P > c ? (P - c + num_caches - 1) / num_caches : 0;
    for (int64_t g0 = 0; g0 < count; g0 += resident) {
      const int64_t g1 = g0 + resident < count ? g0 + resident : count;
      for (int64_t it = 0;; ++it) {
        group.clear();
        for (int64_t j = g0; j < g1; ++j) {
          const int64_t t = c + j * num_caches + it * P;
          if (t >= T) continue;
          int m = 0, n = 0;
          order_tile(o, static_cast<int>(t), m, n);
          const int64_t row0 = static_cast<int64_t>(m) * r.bm, col0 = static_cast<int64_t>(n) * r.bn;
          group.push_back({row0, std::min(r.M, row0 + r.bm), col0, std::min(r.N, col0 + r.bn)});
        }
        if (group.empty()) break;
        for (int64_t kb = 0; kb < nk; ++kb) {
          const int64_t k0 = kb * r.bk, k1 = std::min(r.K, k0 + r.bk);
          for (const Tile& tl : group) {
            for (int64_t row = tl.row0; row < tl.row1; ++row)
              cache.read_range(r.a_base + (static_cast<uint64_t>(row) * r.K + k0) * e, (k1 - k0) * r.elem_bytes);
            for (int64_t k = k0; k < k1; ++k)
              cache.read_range(r.b_base + (static_cast<uint64_t>(k) * r.N + tl.col0) * e,
                               (tl.col1 - tl.col0) * r.elem_bytes);
          }
        }
      }
    }
    *hits += cache.hits;
    *accesses += cache.accesses;
  }
}

}  // namespace tbl
