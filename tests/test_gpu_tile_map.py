"""GPU parity: tbl_tile_map tables equal the oracle's, bit for bit, for every order, group size,
remap flag and grid (the pages' 8x8 / 4x4 grids, the workloads' 8x8, 16x16, 32x32 and 40x24
grids, odd rectangular grids and a large one)."""

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
