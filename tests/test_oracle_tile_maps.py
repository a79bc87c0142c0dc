"""Pins of the tile-order oracle against what the pages print and what the mathematics fixes.

CPU only. Pins used:
  * the four 8x8 tables of "CUDA Thread Block Swizzle" (sections "Linear Swizzle",
    "Grouped 2D Panel Swizzle", "Morton / Z-order Swizzle", "Bitwise XOR Swizzle");
  * the 4x4 group-major and serpentine tables, "Example 1" (per-cluster work lists, ownership
    grid, tile sequences of clusters 1 and 2) and "Example 2" (cluster tile -> CTA tile by rank) of
    the tvm_tirx ClusterPersistentScheduler2D page; clusters of g tile rows over a row-major
    cluster grid reproduce the printed group-major table;
  * special cases: panel g=1 is row-major, panel g >= grid rows is column-major, serpentine with
    s >= grid columns is row-major, serpentine s=1 is the column boustrophedon;
  * explicit walks (nested loops that place ids one by one) for panel and serpentine;
  * bijectivity by brute force, and the remap's hand-computed values.
"""

import itertools

import numpy as np
import pytest

from conftest import golden_grid, golden_sections, golden_lines
from oracle import tile_maps as tm


def _printed(mode, gm, gn, group=1):
    m, n = tm.tile_table(mode, gm, gn, group)
    return tm.inverse_grid(m, n, gm, gn)


@pytest.mark.parametrize("fixture,mode,group", [
    ("p1_row_major_8x8.txt", tm.ROW, 1),
    ("p1_panel_g4_8x8.txt", tm.PANEL, 4),
    ("p1_morton_8x8.txt", tm.MORTON, 1),
    ("p1_xor_8x8.txt", tm.XOR, 1),
])
def test_page1_8x8_tables(fixture, mode, group):
    assert np.array_equal(_printed(mode, 8, 8, group), golden_grid(fixture))


def test_page3_group_major_4x4():
    assert np.array_equal(_printed(tm.PANEL, 4, 4, 2), golden_grid("p3_group_major_4x4_g2.txt"))


def test_page3_serpentine_4x4():
    assert np.array_equal(_printed(tm.SERPENTINE, 4, 4, 2), golden_grid("p3_serpentine_4x4_s2.txt"))


def test_page3_example1_clusters():
    sec = golden_sections("p3_example1_clusters.txt")
    gm = gn = 4
    P = 3
    T = gm * gn
    for ln in sec["work"][1]:
        c, _, ids = ln.partition(":")
        assert tm.program_tiles(int(c), P, T) == [int(v) for v in ids.split()]
    owner = np.array([[int(v) for v in ln.split()] for ln in sec["owner"][1]])
    m, n = tm.tile_table(tm.PANEL, gm, gn, 2)
    got = np.full((gm, gn), -1)
    for c in range(P):
        for t in tm.program_tiles(c, P, T):
            got[m[t], n[t]] = c
    assert np.array_equal(got, owner)
    for ln in sec["sequence"][1]:
        c, _, seq = ln.partition(":")
        want = [tuple(int(v) for v in pair.split(",")) for pair in seq.split()]
        have = [(int(m[t]), int(n[t])) for t in tm.program_tiles(int(c), P, T)]
        assert have == want


GRIDS = [(1, 1), (1, 7), (7, 1), (3, 5), (8, 8), (16, 16), (40, 24), (24, 40), (12, 12), (5, 13),
         (32, 32), (13, 64)]


@pytest.mark.parametrize("gm,gn", GRIDS)
def test_panel_special_cases(gm, gn):
    r = tm.tile_table(tm.ROW, gm, gn)
    c = tm.tile_table(tm.COL, gm, gn)
    p1 = tm.tile_table(tm.PANEL, gm, gn, 1)
    assert np.array_equal(p1[0], r[0]) and np.array_equal(p1[1], r[1])
    for g in (gm, gm + 1, 4 * gm + 3):
        pg = tm.tile_table(tm.PANEL, gm, gn, g)
        assert np.array_equal(pg[0], c[0]) and np.array_equal(pg[1], c[1])


@pytest.mark.parametrize("gm,gn", GRIDS)
def test_serpentine_special_cases(gm, gn):
    r = tm.tile_table(tm.ROW, gm, gn)
    for s in (gn, gn + 5):
        sg = tm.tile_table(tm.SERPENTINE, gm, gn, s)
        assert np.array_equal(sg[0], r[0]) and np.array_equal(sg[1], r[1])
    # s = 1: one column at a time, alternately downwards and upwards
    m, n = tm.tile_table(tm.SERPENTINE, gm, gn, 1)
    walk = [(i if col % 2 == 0 else gm - 1 - i, col) for col in range(gn) for i in range(gm)]
    assert [(int(a), int(b)) for a, b in zip(m, n)] == walk


def _panel_walk(gm, gn, g):
    """Place ids by walking groups of g rows, column by column, top to bottom."""
    out = []
    for first in range(0, gm, g):
        rows = list(range(first, min(first + g, gm)))
        for col in range(gn):
            for row in rows:
                out.append((row, col))
    return out


def _serpentine_walk(gm, gn, s):
    out = []
    for k, first in enumerate(range(0, gn, s)):
        cols = list(range(first, min(first + s, gn)))
        rows = range(gm) if k % 2 == 0 else range(gm - 1, -1, -1)
        for row in rows:
            for col in cols:
                out.append((row, col))
    return out


@pytest.mark.parametrize("gm,gn,g", [(8, 8, 4), (8, 8, 2), (16, 16, 8), (32, 32, 8), (40, 24, 8),
                                     (40, 24, 16), (4, 4, 2), (12, 5, 3), (64, 64, 16), (6, 9, 3)])
def test_panel_matches_walk_when_groups_align(gm, gn, g):
    # Page 1's row formula (id mod the group's height) equals a plain top-to-bottom walk whenever
    # the last group starts at an id divisible by its height; all these grids have that property.
    m, n = tm.tile_table(tm.PANEL, gm, gn, g)
    assert [(int(a), int(b)) for a, b in zip(m, n)] == _panel_walk(gm, gn, g)


def test_panel_partial_group_rotation():
    # gm=5, g=3: last group (rows 3..4) starts at id 15, which is odd, so page 1's formula puts
    # id 15 on row 3 + 15 mod 2 = 4 and id 16 on row 3: the walk's column order rotated by one.
    m, n = tm.tile_table(tm.PANEL, 5, 5, 3)
    assert (int(m[15]), int(n[15])) == (4, 0)
    assert (int(m[16]), int(n[16])) == (3, 0)
    assert tm.is_bijective(m, n, 5, 5)


@pytest.mark.parametrize("gm,gn,s", [(4, 4, 2), (8, 8, 2), (32, 32, 8), (40, 24, 8), (40, 24, 16),
                                     (7, 10, 3), (16, 16, 16), (9, 4, 3)])
def test_serpentine_matches_walk(gm, gn, s):
    m, n = tm.tile_table(tm.SERPENTINE, gm, gn, s)
    assert [(int(a), int(b)) for a, b in zip(m, n)] == _serpentine_walk(gm, gn, s)


@pytest.mark.parametrize("gm,gn", GRIDS)
def test_panel_serpentine_always_bijective(gm, gn):
    for g in (1, 2, 3, 4, 8, 16, 64):
        assert tm.is_bijective(*tm.tile_table(tm.PANEL, gm, gn, g), gm, gn)
        assert tm.is_bijective(*tm.tile_table(tm.SERPENTINE, gm, gn, g), gm, gn)
    assert tm.is_bijective(*tm.tile_table(tm.ROW, gm, gn), gm, gn)
    assert tm.is_bijective(*tm.tile_table(tm.COL, gm, gn), gm, gn)


@pytest.mark.parametrize("p", range(0, 11))
def test_morton_xor_bijective_on_square_powers_of_two(p):
    g = 2 ** p
    for mode in (tm.MORTON, tm.XOR):
        assert tm.is_bijective(*tm.tile_table(mode, g, g), g, g)


def test_morton_xor_not_bijective_off_powers_of_two():
    for gm, gn in [(12, 12), (40, 24), (8, 16)]:
        for mode in (tm.MORTON, tm.XOR):
            assert not tm.is_bijective(*tm.tile_table(mode, gm, gn), gm, gn)


def test_morton_inverse_interleave():
    # On a 2^p square grid Z-order places tile (m, n) at the id whose even bits spell m and odd
    # bits spell n; build that id from (m, n) and compare with the forward table.
    g = 64
    m, n = tm.tile_table(tm.MORTON, g, g)
    for t in range(g * g):
        mm, nn = int(m[t]), int(n[t])
        rebuilt = sum(((mm >> i) & 1) << (2 * i) for i in range(6)) + \
            sum(((nn >> i) & 1) << (2 * i + 1) for i in range(6))
        assert rebuilt == t


def test_xcd_remap_values_and_permutation():
    assert [tm.xcd_remap(t, 64, 8) for t in (0, 1, 8, 9, 63)] == [0, 8, 1, 9, 63]
    for T in list(range(1, 300)) + [960, 1024, 4096]:
        t = np.arange(T)
        r = tm.xcd_remap(t, T, 8)
        assert np.array_equal(np.sort(r), t)
        T8 = 8 * (T // 8)
        assert np.array_equal(r[T8:], t[T8:])
        # domain d = t mod 8 receives a contiguous block of the order, in dispatch order
        for d in range(8):
            block = r[:T8][t[:T8] % 8 == d]
            assert np.array_equal(block, np.arange(d * (T8 // 8), (d + 1) * (T8 // 8)))


def test_remap_flag_composes_with_order():
    gm = gn = 16
    base_m, base_n = tm.tile_table(tm.PANEL, gm, gn, 4)
    m, n = tm.tile_table(tm.PANEL | tm.XCD_REMAP, gm, gn, 4)
    r = tm.xcd_remap(np.arange(gm * gn), gm * gn, 8)
    assert np.array_equal(m, base_m[r]) and np.array_equal(n, base_n[r])


def test_program_tiles_cover_every_id_once():
    for T, P in itertools.product((1, 7, 64, 960, 1024), (1, 3, 8, 192, 256, 2000)):
        seen = sorted(t for p in range(P) for t in tm.program_tiles(p, P, T))
        assert seen == list(range(T))


# ---- the two-level (cluster) schedule of page 3 ----

def test_page3_example2_cluster_expansion():
    sec = golden_sections("p3_example2_cluster_expansion.txt")
    mt, nt, cm, cn, cgm, cgn = (int(v) for v in sec["grid"][1][0].split())
    assert (mt // cm, nt // cn) == (cgm, cgn)
    for ln in sec["expand"][1]:
        lhs, _, rhs = ln.partition(":")
        tile, rank = lhs.split()
        mi, ni = (int(v) for v in tile.split(","))
        want = tuple(int(v) for v in rhs.split(","))
        assert tm.cluster_expand(mi, ni, int(rank), cm, cn) == want
    # the same through the full map: the CTA index t = cluster * CLUSTER_SIZE + rank of a cluster
    # whose work index the scheduler maps to tile (1, 2) (row-major over the 4 x 4 cluster grid: 6)
    m, n = tm.tile_table(tm.ROW, mt, nt, cluster=(cm, cn))
    assert (m[6 * 2], n[6 * 2]) == (2, 2) and (m[6 * 2 + 1], n[6 * 2 + 1]) == (3, 2)


def test_clusters_of_rows_over_row_major_are_group_major():
    # clusters of g tile rows handed out in row-major order walk g rows column by column: page 3's
    # group-major order, whose 4x4 table the page prints
    m, n = tm.tile_table(tm.ROW, 4, 4, cluster=(2, 1))
    assert np.array_equal(tm.inverse_grid(m, n, 4, 4), golden_grid("p3_group_major_4x4_g2.txt"))
    for gm, gn, g in [(8, 8, 4), (12, 5, 3), (16, 16, 8), (6, 9, 2)]:
        assert np.array_equal(np.stack(tm.tile_table(tm.ROW, gm, gn, cluster=(g, 1))),
                              np.stack(tm.tile_table(tm.PANEL, gm, gn, g)))


@pytest.mark.parametrize("mode,group", [(tm.ROW, 1), (tm.COL, 1), (tm.PANEL, 2), (tm.PANEL, 3),
                                        (tm.SERPENTINE, 2), (tm.MORTON, 1), (tm.XOR, 1)])
def test_unit_clusters_are_the_plain_order(mode, group):
    for gm, gn in [(4, 4), (8, 8), (6, 10), (16, 16)]:
        if mode in (tm.MORTON, tm.XOR) and gm != gn:
            continue
        for flags in (mode, mode | tm.XCD_REMAP):
            assert np.array_equal(np.stack(tm.tile_table(flags, gm, gn, group, cluster=(1, 1))),
                                  np.stack(tm.tile_table(flags, gm, gn, group)))
            assert np.array_equal(np.stack(tm.tile_table(flags, gm, gn, group, cluster=(1, 1))),
                                  np.stack(tm.clustered(mode, tm.xcd_remap(np.arange(gm * gn), gm * gn)
                                                        if flags & tm.XCD_REMAP else np.arange(gm * gn),
                                                        gm, gn, group, 1, 1)))


@pytest.mark.parametrize("cm,cn", [(2, 1), (1, 2), (2, 2), (4, 2), (3, 1)])
@pytest.mark.parametrize("mode,group", [(tm.ROW, 1), (tm.COL, 1), (tm.PANEL, 2), (tm.SERPENTINE, 3),
                                        (tm.MORTON, 1), (tm.XOR, 1)])
def test_clustered_orders_bijective_and_blockwise(mode, group, cm, cn):
    for cgm, cgn in [(4, 4), (8, 8), (5, 7), (16, 16)]:
        if mode in (tm.MORTON, tm.XOR) and (cgm != cgn or cgm & (cgm - 1)):
            continue
        gm, gn = cgm * cm, cgn * cn
        for flags in (mode, mode | tm.XCD_REMAP):
            m, n = tm.tile_table(flags, gm, gn, group, cluster=(cm, cn))
            assert tm.is_bijective(m, n, gm, gn)
            # without the remap, every run of cm*cn consecutive ids covers one aligned cluster block,
            # rank r at offset (r mod cm, r div cm)
            if flags & tm.XCD_REMAP:
                continue
            cs = cm * cn
            for c in range(gm * gn // cs):
                mm, nn = m[c * cs:(c + 1) * cs], n[c * cs:(c + 1) * cs]
                assert np.all(mm // cm == mm[0] // cm) and np.all(nn // cn == nn[0] // cn)
                assert np.array_equal(mm % cm, np.arange(cs) % cm)
                assert np.array_equal(nn % cn, np.arange(cs) // cm)


def test_clustered_rejects_partial_clusters():
    with pytest.raises(ValueError):
        tm.clustered(tm.ROW, np.arange(15), 5, 3, 1, 2, 1)
