/*
 * Oracle -- TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
 * leg may load this file's library; the product library shares no code with it.
 *
 * The GEMM's operand reads replayed cache line by cache line through set-associative LRU caches.
 *
 * Source: "CUDA Thread Block Swizzle" (leimao.github.io), section "CUDA Thread Block Swizzle
 * Benchmark". Its offline predictor replays the reads of the tiles that run together, k block by k
 * block, each tile reading its A block and then its B block, through one least-recently-used cache,
 * and predicts the hit rate as hits over reads. This file keeps that replay order and changes what
 * is counted and what holds it, a reading for a GPU whose L2 is split per XCD and indexed by address:
 *
 *   - The unit of a read is a cache line of `line_bytes`, not a whole operand block. At k block j a
 *     tile reads, for every A row it covers (rows < M), the bytes of k = j*bk .. j*bk+bk-1 (k < K),
 *     and then, for every B row k of the block (k < K), the bytes of its columns (< N). Each read of
 *     a contiguous byte range counts one access per line the range touches.
 *   - Each cache has `sets` sets of `ways` lines and is least-recently-used within a set. Line L
 *     (byte address / line_bytes) lives in set (L xor ((L >> fold_from) mod 2^fold_width)) mod sets:
 *     the set index is the line number's low bits with one higher bit-field folded onto its lowest
 *     bits. fold_width = 0 is the plain modulo.
 *   - Placement and grouping as the XCD-aware block replay: program p runs tile ids p, p + P, ...;
 *     it runs on cache p mod num_caches; a cache runs its programs `resident` at a time in program
 *     order, and each loop iteration of such a group is one set of tiles read together, k block by
 *     k block, tiles in program order, A before B.
 *
 * Output: hits, accesses, and misses (every miss fills one whole line, so fetched bytes are
 * misses x line_bytes).
 *
 * Written for a reader to check, not for speed: one set is an array of line numbers, most recently
 * used first; a hit moves its line to the front, a miss shifts the array down by one (dropping the
 * last line when the set is full) and puts the new line in front.
 */
#include <stdint.h>
#include <stdlib.h>

int64_t oracle_l2_set_of(int64_t line, int64_t sets, int fold_from, int fold_width) {
  int64_t folded = fold_width > 0 ? (line >> fold_from) & ((INT64_C(1) << fold_width) - 1) : 0;
  return (line ^ folded) % sets;
}

typedef struct {
  int64_t sets;
  int ways;
  int fold_from, fold_width;
  int64_t line_bytes;
  int64_t* lines;  /* sets x ways line numbers, -1 for an empty way; most recent first */
  int64_t hits, accesses;
} Cache;

static void cache_read_line(Cache* c, int64_t line) {
  int64_t* way = c->lines + oracle_l2_set_of(line, c->sets, c->fold_from, c->fold_width) * c->ways;
  int pos = 0;
  while (pos < c->ways && way[pos] != line) ++pos;
  c->accesses += 1;
  if (pos < c->ways) {
    c->hits += 1;
  } else {
    pos = c->ways - 1;  /* a miss: the last way's line (or the empty marker) is dropped */
  }
  for (int i = pos; i > 0; --i) way[i] = way[i - 1];
  way[0] = line;
}

/* one access per line that bytes [first, first + count) touch */
static void cache_read_range(Cache* c, int64_t first, int64_t count) {
  if (count <= 0) return;
  for (int64_t line = first / c->line_bytes; line <= (first + count - 1) / c->line_bytes; ++line)
    cache_read_line(c, line);
}

static int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

/* The reads of tile (m, n) at k block j. */
static void read_tile_step(Cache* c, int64_t m, int64_t n, int64_t j, int64_t M, int64_t N, int64_t K,
                           int elem_bytes, int bm, int bn, int bk, int64_t a_base, int64_t b_base) {
  const int64_t k0 = j * bk, k1 = min64(K, k0 + bk);
  for (int64_t row = m * bm; row < min64(M, m * bm + bm); ++row)
    cache_read_range(c, a_base + (row * K + k0) * elem_bytes, (k1 - k0) * elem_bytes);
  const int64_t n0 = n * bn, n1 = min64(N, n0 + bn);
  for (int64_t k = k0; k < k1; ++k)
    cache_read_range(c, b_base + (k * N + n0) * elem_bytes, (n1 - n0) * elem_bytes);
}

/*
 * tile_m, tile_n: the order's table (tile id -> m, n), T entries. Returns 0, or -1 for arguments
 * out of range or a failed allocation. out[0] = hits, out[1] = accesses, out[2] = misses.
 */
int oracle_l2_lines(const int64_t* tile_m, const int64_t* tile_n, int64_t T, int64_t M, int64_t N,
                    int64_t K, int elem_bytes, int bm, int bn, int bk, int num_caches,
                    int64_t num_programs, int resident, int64_t sets, int ways, int64_t line_bytes,
                    int fold_from, int fold_width, int64_t a_base, int64_t b_base, int64_t* out) {
  if (T < 0 || M < 1 || N < 1 || K < 1 || elem_bytes < 1 || bm < 1 || bn < 1 || bk < 1 ||
      num_caches < 1 || num_programs < 0 || resident < 1 || sets < 1 || ways < 1 || line_bytes < 1 ||
      fold_from < 0 || fold_from > 62 || fold_width < 0 || fold_width > 62 || a_base < 0 || b_base < 0)
    return -1;
  const int64_t P = num_programs == 0 ? T : num_programs;
  const int64_t nk = (K + bk - 1) / bk;
  out[0] = out[1] = out[2] = 0;
  for (int x = 0; x < num_caches; ++x) {
    Cache c = {sets, ways, fold_from, fold_width, line_bytes, NULL, 0, 0};
    c.lines = (int64_t*)malloc(sizeof(int64_t) * (size_t)(sets * ways));
    if (c.lines == NULL) return -1;
    for (int64_t i = 0; i < sets * ways; ++i) c.lines[i] = -1;
    /* this cache's programs: x, x + num_caches, ... < P */
    const int64_t count = P > x ? (P - x + num_caches - 1) / num_caches : 0;
    for (int64_t g0 = 0; g0 < count; g0 += resident) {
      const int64_t g1 = min64(count, g0 + resident);
      for (int64_t it = 0;; ++it) {
        int any = 0;
        for (int64_t j = 0; j < nk; ++j)
          for (int64_t q = g0; q < g1; ++q) {
            const int64_t t = x + q * num_caches + it * P;
            if (t >= T) continue;
            any = 1;
            read_tile_step(&c, tile_m[t], tile_n[t], j, M, N, K, elem_bytes, bm, bn, bk, a_base, b_base);
          }
        if (!any) break;
      }
    }
    out[0] += c.hits;
    out[1] += c.accesses;
    out[2] += c.accesses - c.hits;
    free(c.lines);
  }
  return 0;
}
