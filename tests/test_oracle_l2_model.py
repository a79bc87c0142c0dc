"""Pins for the oracle's offline L2 model ("CUDA Thread Block Swizzle", section "CUDA Thread Block
Swizzle Benchmark").

  * the page's printed run: the 11 predicted hit rates of the 8192^3, 128x128x32 fp16 sweep at 64 MB
    and concurrency 168, and the two Spearman values computed from its printed columns;
  * the LRU against a brute-force list-based LRU on small random traces (including blocks of two
    sizes and a block larger than the whole cache, which the model keeps as the only entry);
  * a closed form: with unbounded capacity every distinct block misses exactly once;
  * Spearman against scipy where there are no ties, and its index-order tie rule on a hand case;
  * the XCD variant reduces to the page's model with one XCD.
"""

import numpy as np
import pytest
import scipy.stats

from conftest import golden_lines
from oracle import l2_model, tile_maps as tm

# the printed run: 8192^3 fp16 with 128x128x32 tiles -> 64x64 tiles, 256 k blocks of 8 KiB each
GRID, GRID_K, BLOCK_BYTES, CAPACITY, CONCURRENCY = 64, 256, 128 * 32 * 2, 64 * 1024 * 1024, 168


def _fixture():
    rows, spearman = [], {}
    for ln in golden_lines("p1_predicted_l2_hit_rates.txt"):
        tok = ln.split()
        if tok[0] == "spearman":
            spearman[tok[1]] = float(tok[2])
        else:
            rows.append((tok[0], int(tok[1]), int(tok[2]), float(tok[3]), float(tok[4]), float(tok[5])))
    return rows, spearman


ROWS, SPEARMAN = _fixture()


@pytest.mark.parametrize("name,mode,group,printed", [(r[0], r[1], r[2], r[3]) for r in ROWS])
def test_printed_predicted_hit_rates(name, mode, group, printed):
    m, n = tm.tile_table(mode, GRID, GRID, group)
    pred = l2_model.predict_hit_rate(m, n, GRID_K, BLOCK_BYTES, BLOCK_BYTES, CAPACITY, CONCURRENCY)
    assert abs(pred - printed) <= 0.005, (name, pred, printed)


def test_printed_spearman_values():
    pred = [r[3] for r in ROWS]
    assert round(l2_model.rank_correlation(pred, [r[4] for r in ROWS]), 3) == SPEARMAN["nonpersistent"]
    assert round(l2_model.rank_correlation(pred, [r[5] for r in ROWS]), 3) == SPEARMAN["persistent"]


def _brute_lru(trace, capacity):
    """A list-based LRU: most recent entry last, eviction from the front while over capacity and more
    than one entry is held."""
    held, hits = [], 0
    for key, size in trace:
        found = [i for i, (k, _) in enumerate(held) if k == key]
        if found:
            hits += 1
            held.append(held.pop(found[0]))
            continue
        held.append((key, size))
        while sum(s for _, s in held) > capacity and len(held) > 1:
            held.pop(0)
    return hits


@pytest.mark.parametrize("seed", range(6))
def test_lru_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    keys = [("A", int(i)) for i in range(12)] + [("B", int(i)) for i in range(12)]
    size = {k: (3 if k[0] == "A" else 5) for k in keys}
    size[("A", 0)] = 100  # larger than the cache: kept alone until the next miss
    capacity = int(rng.integers(8, 40))
    trace = [(keys[int(i)], size[keys[int(i)]]) for i in rng.integers(0, len(keys), 400)]
    cache = l2_model.ByteLRU(capacity)
    for key, sz in trace:
        cache.access(key, sz)
    assert cache.hits == _brute_lru(trace, capacity)
    assert cache.hits + cache.misses == len(trace)
    assert cache.bytes_held <= max(capacity, max(sz for _, sz in trace))


def test_oversize_block_is_kept_alone():
    cache = l2_model.ByteLRU(10)
    cache.access("big", 50)
    assert list(cache.held) == ["big"] and cache.bytes_held == 50
    cache.access("big", 50)
    assert cache.hits == 1
    cache.access("small", 4)
    assert list(cache.held) == ["small"] and cache.bytes_held == 4


@pytest.mark.parametrize("mode,group", [(tm.ROW, 1), (tm.PANEL, 3), (tm.SERPENTINE, 2), (tm.COL, 1)])
@pytest.mark.parametrize("gm,gn,gk", [(5, 7, 3), (8, 8, 4)])
def test_unbounded_cache_misses_each_block_once(mode, group, gm, gn, gk):
    m, n = tm.tile_table(mode, gm, gn, group)
    for conc in (1, 4, gm * gn):
        pred = l2_model.predict_hit_rate(m, n, gk, 16, 16, 1 << 40, conc)
        # distinct blocks: A (m, k) for every tile row and k, B (k, n) for every tile column and k
        misses = gm * gk + gn * gk
        accesses = 2 * gm * gn * gk
        assert pred == pytest.approx(100.0 * (accesses - misses) / accesses, abs=1e-12)


def test_one_block_cache_hits_nothing_but_repeats():
    # with room for one block, only an immediately repeated block hits: on a 1-column grid the B block
    # (k, 0) never repeats back to back, and A (m, k) is followed by B, so nothing hits
    m, n = tm.tile_table(tm.ROW, 4, 1, 1)
    assert l2_model.predict_hit_rate(m, n, 3, 8, 8, 8, 4) == 0.0


@pytest.mark.parametrize("seed", range(4))
def test_rank_correlation_matches_scipy_without_ties(seed):
    rng = np.random.default_rng(100 + seed)
    x, y = rng.permutation(17).astype(float), rng.normal(size=17)
    assert l2_model.rank_correlation(x, y) == pytest.approx(scipy.stats.spearmanr(x, y)[0], abs=1e-12)


def test_rank_correlation_ties_keep_index_order():
    # x ties all but its last entry: ranks 0,1,2 in index order then 3, so x ranks like y = 0,1,2,3
    assert l2_model.rank_correlation([1.0, 1.0, 1.0, 2.0], [0.0, 1.0, 2.0, 3.0]) == pytest.approx(1.0)
    # averaged ranks (1, 1, 1, 3) would give 3 / sqrt(3 * 5); the index rule differs from scipy's
    assert scipy.stats.spearmanr([1.0, 1.0, 1.0, 2.0], [0.0, 1.0, 2.0, 3.0])[0] == pytest.approx(
        np.sqrt(3 / 5))
    assert l2_model.rank_correlation([1.0, 2.0, 3.0], [5.0, 5.0, 5.0]) == pytest.approx(1.0)
    assert l2_model.rank_correlation([1.0], [2.0]) == 0.0


@pytest.mark.parametrize("mode,group", [(tm.ROW, 1), (tm.PANEL, 4), (tm.MORTON, 1)])
def test_xcd_variant_with_one_xcd_is_the_page_model(mode, group):
    gm = gn = 16
    m, n = tm.tile_table(mode, gm, gn, group)
    cap, gk, conc = 40 * 64, 8, 24
    page = l2_model.predict_hit_rate(m, n, gk, 64, 64, cap, conc)
    # non-persistent: one program per tile, resident in program order
    assert l2_model.predict_hit_rate_xcd(m, n, gk, 64, 64, cap, gm * gn, conc, num_xcds=1) == \
        pytest.approx(page, abs=1e-12)
    # persistent: P = concurrency programs step through tile ids it*P .. it*P + P - 1 together
    assert l2_model.predict_hit_rate_xcd(m, n, gk, 64, 64, cap, conc, conc, num_xcds=1) == \
        pytest.approx(page, abs=1e-12)


def test_xcd_variant_splits_programs_round_robin():
    # 8 XCDs, each holding one block: program p's accesses go only to XCD p mod 8, so with one tile per
    # program and one k block every access is a first touch on its own XCD
    m, n = tm.tile_table(tm.ROW, 4, 4, 1)
    assert l2_model.predict_hit_rate_xcd(m, n, 1, 8, 8, 8, 16, 1) == 0.0
    # with 2 XCDs and unbounded caches, XCD 0 runs the even tile ids (row-major on 4x4: columns 0 and
    # 2 of every row) -> A blocks (m, 0) repeat once per row, B blocks (0, n) once per column pair
    hit = l2_model.predict_hit_rate_xcd(m, n, 1, 8, 8, 1 << 30, 16, 8, num_xcds=2)
    # per XCD: 8 tiles, 16 accesses; distinct blocks 4 A + 2 B -> 10 hits
    assert hit == pytest.approx(100.0 * 20 / 32)
