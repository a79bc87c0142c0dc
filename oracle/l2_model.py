"""Oracle: the offline L2 hit-rate model of "CUDA Thread Block Swizzle" and its rank check, plus
an XCD-aware variant.

TEST INFRASTRUCTURE (see the package docstring): not imported by the library.

Source: "CUDA Thread Block Swizzle" (leimao.github.io), section "CUDA Thread Block Swizzle
Benchmark". What the model computes, restated:
  * the cache is least-recently-used with a capacity counted in bytes; a block that is not held is
    a miss and becomes held; after that, while the held bytes exceed the capacity and more than one
    block is held, the least recently used block leaves;
  * the tiles run in waves of ``concurrency`` consecutive tile ids of the order; inside a wave the
    reads advance k block by k block, and at each k every tile of the wave, in id order, reads its
    A block (m, k) and then its B block (k, n);
  * predicted hit rate = hits / reads.
The page ranks predicted hit rates against measured throughput with a Spearman coefficient (the
Pearson correlation of the ranks) whose equal values are ranked in index order.

``predict_counts_xcd`` is this library's reading for gfx950 (the page models one shared L2): eight
XCDs with private L2s; workgroup p runs on XCD p mod 8, and each XCD replays only its own
workgroups' reads through its own cache.

Written as a read stream (a generator of (block, bytes) in the model's order) fed to a cache that
keeps its blocks in a ring ordered by their last read.
"""

import itertools

import numpy as np


class ByteLRU:
    """LRU cache whose capacity is counted in bytes; blocks may differ in size.

    The held blocks form a ring through two maps, ``newer`` and ``older``, around a sentinel: the
    block after the sentinel in the ``older`` direction is the most recently read, the one before
    it (``newer[sentinel]``) the least recently read. A read unlinks its block and relinks it next
    to the sentinel; an eviction unlinks the block at the other end."""

    _END = object()

    def __init__(self, capacity_bytes):
        self.capacity = capacity_bytes
        self.held = {}                          # block -> bytes
        self.newer = {self._END: self._END}     # block -> the block read after it
        self.older = {self._END: self._END}     # block -> the block read before it
        self.bytes_held = 0
        self.hits = 0
        self.misses = 0

    def _unlink(self, block):
        a, b = self.older.pop(block), self.newer.pop(block)
        self.newer[a], self.older[b] = b, a

    def _link_newest(self, block):
        prev_newest = self.older[self._END]
        self.older[self._END], self.newer[block] = block, self._END
        self.older[block], self.newer[prev_newest] = prev_newest, block

    def read(self, block, nbytes):
        if block in self.held:
            self.hits += 1
            self._unlink(block)
        else:
            self.misses += 1
            self.held[block] = nbytes
            self.bytes_held += nbytes
        self._link_newest(block)
        while self.bytes_held > self.capacity and len(self.held) > 1:
            oldest = self.newer[self._END]
            self._unlink(oldest)
            self.bytes_held -= self.held.pop(oldest)

    # the name the rest of the oracle and its tests use
    access = read

    def hit_rate_pct(self):
        return _pct(self.hits, self.hits + self.misses)


def _wave_reads(wave_tiles, grid_k, a_bytes, b_bytes):
    """The reads of one group of concurrently running tiles: k outermost, then the tiles in order,
    A before B."""
    for k, (m, n), operand in itertools.product(range(grid_k), wave_tiles, ("A", "B")):
        yield ((operand, m, k), a_bytes) if operand == "A" else ((operand, k, n), b_bytes)


def _run(cache, reads):
    for block, nbytes in reads:
        cache.read(block, nbytes)
    return cache


def predict_counts(tile_m, tile_n, grid_k, a_bytes, b_bytes, capacity_bytes, concurrency):
    """Page 1's model as (hits, reads). tile_m / tile_n: the forward table (tile id -> m, n)."""
    tiles = list(zip(np.asarray(tile_m).tolist(), np.asarray(tile_n).tolist()))
    waves = (tiles[w:w + concurrency] for w in range(0, len(tiles), concurrency))
    cache = _run(ByteLRU(capacity_bytes),
                 itertools.chain.from_iterable(_wave_reads(w, grid_k, a_bytes, b_bytes) for w in waves))
    return cache.hits, cache.hits + cache.misses


def predict_hit_rate(tile_m, tile_n, grid_k, a_bytes, b_bytes, capacity_bytes, concurrency):
    """Page 1's model: the predicted hit rate in percent."""
    return _pct(*predict_counts(tile_m, tile_n, grid_k, a_bytes, b_bytes, capacity_bytes,
                                concurrency))


def _pct(hits, reads):
    return 100.0 * hits / reads if reads else 0.0


def _xcd_groups(T, P, x, num_xcds, resident):
    """Tile-id groups that XCD x runs together: its programs x, x + 8, ... taken ``resident`` at a
    time in program order; a group steps through its loop iterations together (program p's
    iteration i is tile p + i P), each iteration one group of concurrently read tiles."""
    programs = np.arange(x, P, num_xcds)
    for start in range(0, len(programs), resident):
        group = programs[start:start + resident]
        for i in itertools.count():
            ids = group + i * P
            ids = ids[ids < T]
            if ids.size == 0:
                break
            yield ids


def predict_counts_xcd(tile_m, tile_n, grid_k, a_bytes, b_bytes, capacity_per_xcd, num_programs,
                       resident_per_xcd, num_xcds=8):
    """XCD-aware variant (a reading; see the module docstring), as (hits, reads) over all XCDs.

    Programs p = 0 .. num_programs-1 run tile ids p, p + P, ... (the stride schedule); program p
    runs on XCD p mod num_xcds. Each XCD runs its programs ``resident_per_xcd`` at a time, in
    program order, and its cache sees, for each group of concurrently running programs, the tiles
    of one loop iteration, k block by k block.
    """
    tile_m, tile_n = np.asarray(tile_m), np.asarray(tile_n)
    T = len(tile_m)
    hits = reads = 0
    for x in range(num_xcds):
        cache = ByteLRU(capacity_per_xcd)
        for ids in _xcd_groups(T, num_programs, x, num_xcds, resident_per_xcd):
            tiles = list(zip(tile_m[ids].tolist(), tile_n[ids].tolist()))
            _run(cache, _wave_reads(tiles, grid_k, a_bytes, b_bytes))
        hits += cache.hits
        reads += cache.hits + cache.misses
    return hits, reads


def predict_hit_rate_xcd(tile_m, tile_n, grid_k, a_bytes, b_bytes, capacity_per_xcd, num_programs,
                         resident_per_xcd, num_xcds=8):
    """The XCD-aware variant's hit rate in percent over all XCDs' reads."""
    return _pct(*predict_counts_xcd(tile_m, tile_n, grid_k, a_bytes, b_bytes, capacity_per_xcd,
                                    num_programs, resident_per_xcd, num_xcds))


def rank_correlation(x, y):
    """Spearman coefficient: Pearson correlation of the ranks, equal values ranked in index order
    (a stable sort keeps equal values in index order; its inverse permutation is the rank)."""
    def ranks(v):
        order = np.argsort(np.asarray(v, dtype=np.float64), kind="stable")
        r = np.empty(len(order), dtype=np.float64)
        r[order] = np.arange(len(order))
        return r
    rx, ry = ranks(x), ranks(y)
    if np.all(rx == rx[0]) or np.all(ry == ry[0]):
        return 0.0
    return float(np.corrcoef(rx, ry)[0, 1])
