"""Oracle: the offline L2 hit-rate model of page 1 and its rank check, plus an XCD-aware variant.

TEST INFRASTRUCTURE (see the package docstring): not imported by the library.

Source: "CUDA Thread Block Swizzle" (leimao.github.io), section "CUDA Thread Block Swizzle
Benchmark": a byte-capacity LRU cache replays the operand blocks that concurrently running tiles
touch; tiles run in waves of ``concurrency`` consecutive tile ids, and within a wave, k block by
k block, every tile reads its A block (m, k) and then its B block (k, n). A miss inserts the block
and evicts least-recently-used blocks while the cache is over capacity and holds more than one
block. The page ranks the predicted hit rates against measured throughput with a Spearman
coefficient in which ties keep their index order.

``predict_hit_rate_xcd`` is this library's reading for gfx950 (the page models one shared L2):
eight XCDs with private L2s; workgroup p runs on XCD p mod 8, and each XCD replays only its own
workgroups' accesses through its own cache.
"""

from collections import OrderedDict

import numpy as np


class ByteLRU:
    """LRU cache whose capacity is counted in bytes; blocks may differ in size."""

    def __init__(self, capacity_bytes):
        self.capacity = capacity_bytes
        self.blocks = OrderedDict()      # key -> size; first entry = least recently used
        self.used = 0
        self.hits = 0
        self.misses = 0

    def access(self, key, size):
        if key in self.blocks:
            self.hits += 1
            self.blocks.move_to_end(key)
            return
        self.misses += 1
        self.blocks[key] = size
        self.used += size
        while self.used > self.capacity and len(self.blocks) > 1:
            _, dropped = self.blocks.popitem(last=False)
            self.used -= dropped

    def hit_rate_pct(self):
        total = self.hits + self.misses
        return 100.0 * self.hits / total if total else 0.0


def _replay(cache, tiles, grid_k, a_bytes, b_bytes):
    for k in range(grid_k):
        for m, n in tiles:
            cache.access(("A", m, k), a_bytes)
            cache.access(("B", k, n), b_bytes)


def predict_counts(tile_m, tile_n, grid_k, a_bytes, b_bytes, capacity_bytes, concurrency):
    """Page 1's model as (hits, accesses). tile_m / tile_n: the forward table (tile id -> m, n)."""
    cache = ByteLRU(capacity_bytes)
    T = len(tile_m)
    for w0 in range(0, T, concurrency):
        wave = list(zip(tile_m[w0:w0 + concurrency].tolist(), tile_n[w0:w0 + concurrency].tolist()))
        _replay(cache, wave, grid_k, a_bytes, b_bytes)
    return cache.hits, cache.hits + cache.misses


def predict_hit_rate(tile_m, tile_n, grid_k, a_bytes, b_bytes, capacity_bytes, concurrency):
    """Page 1's model: the predicted hit rate in percent."""
    return _pct(*predict_counts(tile_m, tile_n, grid_k, a_bytes, b_bytes, capacity_bytes,
                                concurrency))


def _pct(hits, accesses):
    return 100.0 * hits / accesses if accesses else 0.0


def predict_counts_xcd(tile_m, tile_n, grid_k, a_bytes, b_bytes, capacity_per_xcd, num_programs,
                       resident_per_xcd, num_xcds=8):
    """XCD-aware variant (a reading; see the module docstring), as (hits, accesses) over all XCDs.

    Programs p = 0 .. num_programs-1 run tile ids p, p + P, ... (the stride schedule); program p
    runs on XCD p mod num_xcds. Each XCD runs its programs ``resident_per_xcd`` at a time, in
    program order, and its cache sees, for each group of concurrently running programs, the tiles
    of one loop iteration, k block by k block.
    """
    T = len(tile_m)
    P = num_programs
    caches = [ByteLRU(capacity_per_xcd) for _ in range(num_xcds)]
    for x in range(num_xcds):
        programs = list(range(x, P, num_xcds))
        # non-persistent launches (one tile per program) fill the XCD in program order; persistent
        # ones keep the same resident programs and step through their loop iterations together
        for g0 in range(0, len(programs), resident_per_xcd):
            group = programs[g0:g0 + resident_per_xcd]
            it = 0
            while True:
                ids = [p + it * P for p in group if p + it * P < T]
                if not ids:
                    break
                _replay(caches[x], [(int(tile_m[t]), int(tile_n[t])) for t in ids], grid_k,
                        a_bytes, b_bytes)
                it += 1
    return sum(c.hits for c in caches), sum(c.hits + c.misses for c in caches)


def predict_hit_rate_xcd(tile_m, tile_n, grid_k, a_bytes, b_bytes, capacity_per_xcd, num_programs,
                         resident_per_xcd, num_xcds=8):
    """The XCD-aware variant's hit rate in percent over all XCDs' accesses."""
    return _pct(*predict_counts_xcd(tile_m, tile_n, grid_k, a_bytes, b_bytes, capacity_per_xcd,
                                    num_programs, resident_per_xcd, num_xcds))


def rank_correlation(x, y):
    """Spearman coefficient: Pearson correlation of the ranks, ties ranked in index order."""
    def ranks(v):
        order = sorted(range(len(v)), key=lambda i: v[i])   # stable: equal values keep index order
        r = [0.0] * len(v)
        for pos, i in enumerate(order):
            r[i] = float(pos)
        return np.array(r)
    rx, ry = ranks(list(x)), ranks(list(y))
    dx, dy = rx - rx.mean(), ry - ry.mean()
    den = np.sqrt(np.sum(dx * dx) * np.sum(dy * dy))
    return float(np.sum(dx * dy) / den) if den else 0.0
