"""GPU parity: tbl_tile_map tables equal the oracle's, bit for bit, for every order, group size,
remap flag and grid (the pages' 8x8 / 4x4 grids, the workloads' 8x8, 16x16, 32x32 and 40x24
grids, odd rectangular grids, and large grids up to 2^26 ids and the largest accepted dimension)."""

import numpy as np
import pytest
import torch

import thread_block_lds_amd as tbl
from conftest import golden_grid
from oracle import tile_maps as tm

pytestmark = pytest.mark.gpu

GRIDS = [(8, 8), (4, 4), (16, 16), (32, 32), (40, 24), (24, 40), (1, 1), (1, 9), (3, 5), (7, 13),
         (64, 64), (100, 37), (12, 12), (1024, 1024)]
GROUPS = [1, 2, 3, 4, 8, 16, 64, 5000]


def _gpu_table(mode, gm, gn, g):
    m, n, st = tbl.tile_map(mode, gm, gn, g)
    torch.cuda.synchronize()
    return m.cpu().numpy().astype(np.int64), n.cpu().numpy().astype(np.int64), st


@pytest.mark.parametrize("gm,gn", GRIDS)
@pytest.mark.parametrize("remap", [0, tm.XCD_REMAP])
def test_tables_match_oracle(gm, gn, remap):
    for mode in (tm.ROW, tm.COL, tm.PANEL, tm.MORTON, tm.XOR, tm.SERPENTINE):
        groups = GROUPS if mode in (tm.PANEL, tm.SERPENTINE) else [1]
        for g in groups:
            m, n, st = _gpu_table(mode | remap, gm, gn, g)
            om, on = tm.tile_table(mode | remap, gm, gn, g)
            assert np.array_equal(m, om) and np.array_equal(n, on), (mode, remap, gm, gn, g)
            bij = tm.is_bijective(om, on, gm, gn)
            if mode in (tm.MORTON, tm.XOR) and not (gm == gn and gm & (gm - 1) == 0):
                assert st == tbl.WARN_NOT_BIJECTIVE
            else:
                assert st == tbl.OK and bij


@pytest.mark.parametrize("fixture,mode,group,grid", [
    ("p1_row_major_8x8.txt", tm.ROW, 1, 8), ("p1_panel_g4_8x8.txt", tm.PANEL, 4, 8),
    ("p1_morton_8x8.txt", tm.MORTON, 1, 8), ("p1_xor_8x8.txt", tm.XOR, 1, 8),
    ("p3_group_major_4x4_g2.txt", tm.PANEL, 2, 4), ("p3_serpentine_4x4_s2.txt", tm.SERPENTINE, 2, 4),
])
def test_printed_tables_on_gpu(fixture, mode, group, grid):
    m, n, _ = _gpu_table(mode, grid, grid, group)
    assert np.array_equal(tm.inverse_grid(m, n, grid, grid), golden_grid(fixture))


CLUSTER_GRIDS = [(8, 8), (16, 16), (32, 32), (40, 24), (12, 18), (64, 64)]
CLUSTER_SHAPES = [(2, 1), (1, 2), (2, 2), (4, 2), (3, 3), (8, 1)]
CLUSTER_CASES = [(gm, gn, cm, cn) for gm, gn in CLUSTER_GRIDS for cm, cn in CLUSTER_SHAPES
                 if gm % cm == 0 and gn % cn == 0]
CLUSTER_PARTIAL = [(gm, gn, cm, cn) for gm, gn in CLUSTER_GRIDS for cm, cn in CLUSTER_SHAPES
                   if gm % cm or gn % cn]


@pytest.mark.parametrize("gm,gn,cm,cn", CLUSTER_CASES)
def test_cluster_tables_match_oracle(gm, gn, cm, cn):
    cgm, cgn = gm // cm, gn // cn
    for remap in (0, tm.XCD_REMAP):
        for mode in (tm.ROW, tm.COL, tm.PANEL, tm.MORTON, tm.XOR, tm.SERPENTINE):
            for g in ([1, 2, 4, 8] if mode in (tm.PANEL, tm.SERPENTINE) else [1]):
                m, n, st = _gpu_table(mode | remap | tbl.cluster(cm, cn), gm, gn, g)
                om, on = tm.tile_table(mode | remap, gm, gn, g, cluster=(cm, cn))
                assert np.array_equal(m, om) and np.array_equal(n, on), (mode, remap, gm, gn, g, cm, cn)
                if mode in (tm.MORTON, tm.XOR) and not (cgm == cgn and cgm & (cgm - 1) == 0):
                    assert st == tbl.WARN_NOT_BIJECTIVE
                else:
                    assert st == tbl.OK and tm.is_bijective(om, on, gm, gn)


@pytest.mark.parametrize("gm,gn,cm,cn", CLUSTER_PARTIAL)
def test_partial_clusters_rejected(gm, gn, cm, cn):
    """A cluster that does not tile the grid is refused before any launch (as the oracle refuses it)."""
    with pytest.raises(tbl.TblError) as e:
        _gpu_table(tm.ROW | tbl.cluster(cm, cn), gm, gn, 1)
    assert e.value.status == tbl.ERR_SHAPE
    with pytest.raises(ValueError):
        tm.tile_table(tm.ROW, gm, gn, 1, cluster=(cm, cn))


def test_page3_example2_on_gpu():
    # 8 x 4 tiles in 2 x 1 clusters, cluster tiles in row-major order: CTA ids 12 and 13 form the
    # cluster whose scheduler tile is (1, 2); the page's worked case gives them (2, 2) and (3, 2)
    m, n, st = _gpu_table(tm.ROW | tbl.cluster(2, 1), 8, 4, 1)
    assert st == tbl.OK
    assert (m[12], n[12]) == (2, 2) and (m[13], n[13]) == (3, 2)
    # and clusters of 2 rows over row-major reproduce the printed group-major 4x4 table
    m, n, _ = _gpu_table(tm.ROW | tbl.cluster(2, 1), 4, 4, 1)
    assert np.array_equal(tm.inverse_grid(m, n, 4, 4), golden_grid("p3_group_major_4x4_g2.txt"))


@pytest.mark.parametrize("mode,gm,gn,g", [
    (tm.MORTON, 8192, 8192, 1), (tm.MORTON | tm.XCD_REMAP, 8192, 8192, 1), (tm.XOR, 8192, 8192, 1),
    (tm.ROW | tm.XCD_REMAP, 8192, 8192, 1),
    (tm.PANEL, 3000, 5000, 7), (tm.PANEL | tm.XCD_REMAP, 3000, 5000, 7), (tm.SERPENTINE, 3000, 5000, 13),
    (tm.SERPENTINE | tm.XCD_REMAP, 3000, 5000, 13), (tm.COL, 3000, 5000, 1),
    (tm.SERPENTINE, 1 << 20, 3, 2), (tm.PANEL, 3, 1 << 20, 2), (tm.PANEL | tm.XCD_REMAP, 1 << 20, 1, 5),
])
def test_large_tables_match_oracle(mode, gm, gn, g):
    # 2^26 ids at 8192 x 8192 (Morton's and XOR's bit operations on 26-bit ids), 15 M ids with
    # groups and strips that leave partial last groups, and grids at the largest accepted dimension
    m, n, st = _gpu_table(mode, gm, gn, g)
    om, on = tm.tile_table(mode, gm, gn, g)
    assert st == tbl.OK
    assert np.array_equal(m, om) and np.array_equal(n, on), (mode, gm, gn, g)
