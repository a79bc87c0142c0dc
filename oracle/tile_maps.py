"""Oracle: program id -> output tile (m, n) for every tile order, and the persistent schedule.

TEST INFRASTRUCTURE (see the package docstring): not imported by the library.

Every order takes a tile id ``t`` (0 <= t < gm*gn) of a gm x gn output-tile grid and returns the
tile row ``m`` and tile column ``n``. The functions accept Python ints or numpy int64 arrays; numpy
applies the same integer formula elementwise, so a whole table is one call.

Sources:
  [P1] "CUDA Thread Block Swizzle" (leimao.github.io): the four 8x8 tables in sections
       "Linear Swizzle", "Grouped 2D Panel Swizzle", "Morton / Z-order Swizzle" and
       "Bitwise XOR Swizzle", and the CPU pid-mapping functions plus the kernel's tile loop in the
       benchmark script of section "CUDA Thread Block Swizzle Benchmark".
  [P3] "tvm_tirx ... ClusterPersistentScheduler2D" (tvm.apache.org): "Tile Ordering" (group-major),
       "Serpentine Mode", "Example 1: Basic persistent kernel" and "Example 2: 2SM GEMM" (the
       scheduler works on cluster tiles; each CTA of a cluster expands its cluster tile by its rank).

Where the pages are silent or disagree, the reading taken is marked READING below.
"""

import numpy as np

ROW, COL, PANEL, MORTON, XOR, SERPENTINE = 0, 1, 2, 3, 4, 5
XCD_REMAP = 0x100  # flag OR-ed into a mode id
MODE_NAMES = {ROW: "row", COL: "col", PANEL: "panel", MORTON: "morton", XOR: "xor",
              SERPENTINE: "serpentine"}


def row_major(t, gm, gn):
    """[P1] Linear swizzle, row-major: consecutive ids walk along a tile row."""
    return t // gn, t % gn


def col_major(t, gm, gn):
    """[P1] Linear swizzle, column-major: consecutive ids walk down a tile column."""
    return t % gm, t // gm


def panel(t, gm, gn, g):
    """[P1] Grouped 2D panel swizzle with group size g (GROUP_SIZE_M); [P3] group-major order.

    The grid is cut into groups of g tile rows (the last group keeps whatever rows remain). Groups
    are taken in row order; inside a group ids run down a column of the group, then move to the
    next column. The row inside the group is the id modulo the group's actual height, as [P1]'s
    function computes it (not the id's offset inside the group modulo that height; the two differ
    only in a partial last group whose first id is not a multiple of its height).
    """
    ids_per_group = g * gn
    first_m = (t // ids_per_group) * g
    height = np.minimum(gm - first_m, g)
    m = first_m + t % height
    n = (t % ids_per_group) // height
    return m, n


def morton(t, gm, gn):
    """[P1] Morton / Z-order swizzle.

    Bit 2i of the id becomes bit i of m and bit 2i+1 becomes bit i of n, for 16 bit pairs; the
    results are then reduced modulo the grid ([P1] notes this is a bijection only on power-of-two
    grids).
    """
    m = 0 * t
    n = 0 * t
    for i in range(16):
        m = m | (((t >> (2 * i)) & 1) << i)
        n = n | (((t >> (2 * i + 1)) & 1) << i)
    return m % gm, n % gn


def xor(t, gm, gn):
    """[P1] Bitwise XOR swizzle: with x = t mod gn and y = t div gn, m = (x XOR y) mod gm, n = y mod gn."""
    x = t % gn
    y = t // gn
    return (x ^ y) % gm, y % gn


def serpentine(t, gm, gn, s):
    """[P3] Serpentine order with swizzle size s.  READING.

    Read literally, the page's prose (s x s blocks, row-major inside each block) does not produce
    the page's own 4x4 table; the table and its traversal line do fit this reading: the grid is cut
    into column strips s tiles wide (the last strip keeps the remaining columns). Strips are taken
    left to right. Inside strip number k the ids walk the strip's rows, top to bottom when k is even
    and bottom to top when k is odd, and along each strip row the columns ascend.
    """
    per_full_strip = s * gm
    k = t // per_full_strip
    width = np.minimum(s, gn - k * s)
    u = t - k * per_full_strip
    r = u // width
    m = np.where(k % 2 == 0, r, gm - 1 - r)
    n = k * s + u % width
    return m, n


def xcd_remap(t, T, X=8):
    """READING (the pages never mention XCDs).  Tile-id permutation for X private L2 domains.

    Workgroup w runs on domain w mod X (round-robin dispatch), and in the stride schedule the tile
    id t of a program is congruent to the program modulo X whenever X divides the program count.
    The remap gives domain d = t mod X the contiguous block d*(T'/X) ... (d+1)*(T'/X)-1 of the tile
    order, walked in dispatch order, where T' = X*floor(T/X); ids t >= T' are left unchanged.
    """
    T8 = X * (T // X)
    inside = t < T8
    moved = (t % X) * (T8 // X) + t // X
    return np.where(inside, moved, t) if isinstance(t, np.ndarray) else (moved if inside else t)


def order(mode, t, gm, gn, group=1):
    """Apply order ``mode`` (ROW..SERPENTINE) to tile id(s) t. ``group`` is g for PANEL, s for SERPENTINE."""
    if mode == ROW:
        return row_major(t, gm, gn)
    if mode == COL:
        return col_major(t, gm, gn)
    if mode == PANEL:
        return panel(t, gm, gn, group)
    if mode == MORTON:
        return morton(t, gm, gn)
    if mode == XOR:
        return xor(t, gm, gn)
    if mode == SERPENTINE:
        return serpentine(t, gm, gn, group)
    raise ValueError(f"unknown mode {mode}")


def cluster_expand(m_idx, n_idx, rank, cm, cn):
    """[P3] "Example 2": the tile of the CTA with cluster rank ``rank`` in scheduler tile
    (m_idx, n_idx) of a cm x cn cluster: cb_m = rank mod cm, cb_n = rank div cm, and the tile is
    (m_idx * cm + cb_m, n_idx * cn + cb_n)."""
    return m_idx * cm + rank % cm, n_idx * cn + rank // cm


def clustered(mode, t, gm, gn, group, cm, cn):
    """[P3] two-level schedule.  READING (gfx950 has no thread-block clusters).

    Tile id t plays the CTA index of [P3]'s Example 2: its cluster id t div (cm*cn) is the
    scheduler's work index, which ``order`` maps to a scheduler tile (m_idx, n_idx) of the
    (gm/cm) x (gn/cn) cluster-tile grid, and its rank t mod (cm*cn) picks the tile inside that
    cluster tile (``cluster_expand``). cm and cn must divide gm and gn.
    """
    if gm % cm or gn % cn:
        raise ValueError("cluster dimensions must divide the tile grid")
    cs = cm * cn
    m_idx, n_idx = order(mode, t // cs, gm // cm, gn // cn, group)
    return cluster_expand(m_idx, n_idx, t % cs, cm, cn)


def tile_table(mode_flags, gm, gn, group=1, num_xcds=8, cluster=(1, 1)):
    """Forward table: for every tile id t = 0..T-1, the (m, n) it is mapped to (two int64 arrays).

    ``mode_flags`` is a mode id, optionally OR-ed with XCD_REMAP, in which case the id is first
    permuted by ``xcd_remap`` and the order is applied to the permuted id. ``cluster`` = (cm, cn)
    applies the order to cluster tiles and expands them (``clustered``); (1, 1) is the plain order.
    """
    T = gm * gn
    t = np.arange(T, dtype=np.int64)
    if mode_flags & XCD_REMAP:
        t = xcd_remap(t, T, num_xcds)
    cm, cn = cluster
    if (cm, cn) == (1, 1):
        m, n = order(mode_flags & 0xFF, t, gm, gn, group)
    else:
        m, n = clustered(mode_flags & 0xFF, t, gm, gn, group, cm, cn)
    return np.asarray(m, dtype=np.int64), np.asarray(n, dtype=np.int64)


def inverse_grid(m, n, gm, gn):
    """The printed form of a table: a gm x gn grid whose cell (m, n) holds the id mapped there.

    Cells that no id reaches hold -1; if two ids reach one cell the later id wins (callers check
    bijectivity separately)."""
    grid = np.full((gm, gn), -1, dtype=np.int64)
    for t in range(len(m)):
        grid[m[t], n[t]] = t
    return grid


def is_bijective(m, n, gm, gn):
    """True when the table visits every tile of the gm x gn grid exactly once."""
    if len(m) != gm * gn:
        return False
    if np.any(m < 0) or np.any(m >= gm) or np.any(n < 0) or np.any(n >= gn):
        return False
    return len(np.unique(m * gn + n)) == gm * gn


def program_tiles(p, num_programs, T):
    """[P1] kernel tile loop; [P3] "Example 1": program (cluster) p visits ids p, p+P, p+2P, ... < T."""
    return list(range(p, T, num_programs))
