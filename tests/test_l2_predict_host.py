"""tbl_predict_l2 (host code in libtbl.so, no GPU needed) against the oracle's L2 model.

Hit and access counts are integers, so parity is exact. The page's printed predictions are checked
through the library too, for every order of the printed sweep.
"""

import numpy as np
import pytest

import thread_block_lds_amd as tbl
from conftest import golden_lines
from oracle import l2_model, tile_maps as tm


def _printed_rows():
    out = []
    for ln in golden_lines("p1_predicted_l2_hit_rates.txt"):
        tok = ln.split()
        if tok[0] != "spearman":
            out.append((tok[0], int(tok[1]), int(tok[2]), float(tok[3])))
    return out


@pytest.mark.parametrize("name,mode,group,printed", _printed_rows())
def test_library_reproduces_printed_predictions(name, mode, group, printed):
    # 8192^3 fp16, 128x128x32 tiles: 64x64 tiles, 256 k blocks of 8 KiB, 64 MB, waves of 168
    hits, acc, st = tbl.predict_l2(mode, 64, 64, 256, group, 8192, 8192, 64 * 1024 * 1024,
                                   num_caches=1, num_programs=0, resident=168)
    assert st == tbl.OK and acc == 2 * 4096 * 256
    assert abs(100.0 * hits / acc - printed) <= 0.005, (name, 100.0 * hits / acc)


@pytest.mark.parametrize("mode,group", [(tm.ROW, 1), (tm.PANEL, 8), (tm.MORTON, 1)])
def test_library_counts_equal_oracle_on_printed_config(mode, group):
    m, n = tm.tile_table(mode, 64, 64, group)
    want = l2_model.predict_counts(m, n, 256, 8192, 8192, 64 * 1024 * 1024, 168)
    got = tbl.predict_l2(mode, 64, 64, 256, group, 8192, 8192, 64 * 1024 * 1024, 1, 0, 168)[:2]
    assert got == want


def _cases():
    rng = np.random.default_rng(7)
    modes = [tm.ROW, tm.COL, tm.PANEL, tm.MORTON, tm.XOR, tm.SERPENTINE]
    out = []
    for i in range(24):
        mode = modes[i % len(modes)] | (tm.XCD_REMAP if i % 4 == 3 else 0)
        if mode & 0xFF in (tm.MORTON, tm.XOR):
            gm = gn = int(2 ** rng.integers(1, 5))
        else:
            gm, gn = int(rng.integers(1, 19)), int(rng.integers(1, 19))
        group = int(rng.integers(1, 24))
        gk = int(rng.integers(1, 9))
        a_b, b_b = int(rng.choice([16, 24, 64])), int(rng.choice([16, 32, 64]))
        cap = int(rng.integers(0, 40)) * 16
        caches = int(rng.choice([1, 2, 3, 8]))
        programs = int(rng.choice([0, 1, 5, gm * gn, gm * gn + 3, max(1, gm * gn // 3)]))
        resident = int(rng.integers(1, 9))
        out.append((mode, gm, gn, gk, group, a_b, b_b, cap, caches, programs, resident))
    return out


@pytest.mark.parametrize("case", _cases())
def test_library_counts_equal_oracle_xcd_variant(case):
    mode, gm, gn, gk, group, a_b, b_b, cap, caches, programs, resident = case
    m, n = tm.tile_table(mode, gm, gn, group)
    P = programs if programs else gm * gn
    want = l2_model.predict_counts_xcd(m, n, gk, a_b, b_b, cap, P, resident, num_xcds=caches)
    hits, acc, _ = tbl.predict_l2(mode, gm, gn, gk, group, a_b, b_b, cap, caches, programs, resident)
    assert (hits, acc) == want
    assert acc == 2 * gm * gn * gk


def _cluster_cases():
    rng = np.random.default_rng(11)
    modes = [tm.ROW, tm.COL, tm.PANEL, tm.MORTON, tm.XOR, tm.SERPENTINE]
    out = []
    for i in range(24):
        mode = modes[i % len(modes)] | (tm.XCD_REMAP if i % 3 == 2 else 0)
        cm, cn = int(rng.integers(1, 5)), int(rng.integers(1, 4))
        if mode & 0xFF in (tm.MORTON, tm.XOR):
            cgm = cgn = int(2 ** rng.integers(1, 4))
        else:
            cgm, cgn = int(rng.integers(1, 9)), int(rng.integers(1, 9))
        group = int(rng.integers(1, 10))
        caches = int(rng.choice([1, 2, 8]))
        programs = int(rng.choice([0, 3, cgm * cgn * cm * cn + 1]))
        out.append((mode, cm, cn, cgm * cm, cgn * cn, group, caches, programs, int(rng.integers(1, 6))))
    return out


@pytest.mark.parametrize("case", _cluster_cases())
def test_library_counts_equal_oracle_cluster_orders(case):
    # the library evaluates the two-level order with the same code the GEMM runs; the replay only
    # agrees with the oracle's when every tile id lands where the oracle's table puts it
    mode, cm, cn, gm, gn, group, caches, programs, resident = case
    m, n = tm.tile_table(mode, gm, gn, group, cluster=(cm, cn))
    P = programs if programs else gm * gn
    want = l2_model.predict_counts_xcd(m, n, 3, 16, 24, 160, P, resident, num_xcds=caches)
    hits, acc, st = tbl.predict_l2(mode | tbl.cluster(cm, cn), gm, gn, 3, group, 16, 24, 160, caches,
                                   programs, resident)
    assert st == tbl.OK
    assert (hits, acc) == want


def test_cluster_arguments():
    # a cluster that does not tile the grid, and bits above the cluster field
    with pytest.raises(tbl.TblError) as e:
        tbl.predict_l2(tm.ROW | tbl.cluster(2, 1), 5, 4, 1, 1, 8, 8, 64, 1, 0, 1)
    assert e.value.status == tbl.ERR_SHAPE
    with pytest.raises(tbl.TblError) as e:
        tbl.predict_l2(tm.ROW | tbl.cluster(1, 3), 4, 4, 1, 1, 8, 8, 64, 1, 0, 1)
    assert e.value.status == tbl.ERR_SHAPE
    with pytest.raises(tbl.TblError) as e:
        tbl.predict_l2(tm.ROW | (1 << 24), 4, 4, 1, 1, 8, 8, 64, 1, 0, 1)
    assert e.value.status == tbl.ERR_INVALID_ARG
    # Morton on a 4x4 grid of 2x2 clusters: the cluster grid 2x2 is a square power of two
    assert tbl.predict_l2(tm.MORTON | tbl.cluster(2, 2), 4, 4, 1, 1, 8, 8, 64, 1, 0, 1)[2] == tbl.OK
    # ... on a 4x4 grid of 2x1 clusters (a 2x4 cluster grid) it is not
    assert tbl.predict_l2(tm.MORTON | tbl.cluster(2, 1), 4, 4, 1, 1, 8, 8, 64, 1, 0, 1)[2] == tbl.WARN_NOT_BIJECTIVE
    with pytest.raises(ValueError):
        tbl.cluster(0, 1)
    with pytest.raises(ValueError):
        tbl.cluster(1, 17)


def test_not_bijective_order_warns_and_still_predicts():
    hits, acc, st = tbl.predict_l2(tm.XOR, 6, 6, 2, 1, 8, 8, 1 << 20, 1, 0, 4)
    assert st == tbl.WARN_NOT_BIJECTIVE and acc == 2 * 36 * 2
    m, n = tm.tile_table(tm.XOR, 6, 6, 1)
    assert (hits, acc) == l2_model.predict_counts(m, n, 2, 8, 8, 1 << 20, 4)


@pytest.mark.parametrize("kwargs,status", [
    (dict(mode=7), tbl.ERR_INVALID_ARG), (dict(mode=tm.PANEL, group=0), tbl.ERR_INVALID_ARG),
    (dict(grid_m=0), tbl.ERR_SHAPE), (dict(grid_k=0), tbl.ERR_SHAPE),
    (dict(grid_k=(1 << 20) + 1), tbl.ERR_SHAPE), (dict(a_block_bytes=0), tbl.ERR_INVALID_ARG),
    (dict(capacity_bytes=-1), tbl.ERR_INVALID_ARG), (dict(num_caches=0), tbl.ERR_INVALID_ARG),
    (dict(num_caches=65), tbl.ERR_INVALID_ARG), (dict(num_programs=-1), tbl.ERR_INVALID_ARG),
    (dict(resident=0), tbl.ERR_INVALID_ARG),
    # work bound: 2 * T * grid_k > 2^33
    (dict(grid_m=1 << 12, grid_n=1 << 12, grid_k=1 << 10), tbl.ERR_SHAPE),
    # memory bound: (grid_m + grid_n) * grid_k > 2^26
    (dict(grid_m=1 << 16, grid_n=1, grid_k=1 << 11), tbl.ERR_SHAPE),
])
def test_invalid_arguments(kwargs, status):
    args = dict(mode=tm.ROW, grid_m=4, grid_n=4, grid_k=2, group=1, a_block_bytes=8, b_block_bytes=8,
                capacity_bytes=64, num_caches=1, num_programs=0, resident=1)
    args.update(kwargs)
    with pytest.raises(tbl.TblError) as e:
        tbl.predict_l2(**args)
    assert e.value.status == status


# ---- tbl_predict_l2_lines against oracle.l2_lines (exact integer parity) ----

from oracle import l2_lines  # noqa: E402


def _line_cases():
    rng = np.random.default_rng(23)
    modes = [tm.ROW, tm.COL, tm.PANEL, tm.MORTON, tm.XOR, tm.SERPENTINE]
    out = []
    for i in range(30):
        mode = modes[i % len(modes)] | (tm.XCD_REMAP if i % 4 == 1 else 0)
        bm, bn, bk = (int(rng.choice([2, 4, 16, 32])), int(rng.choice([2, 8, 16, 32])),
                      int(rng.choice([1, 4, 8, 32])))
        if mode & 0xFF in (tm.MORTON, tm.XOR):
            g = int(2 ** rng.integers(0, 4))
            M, N = g * bm - int(rng.integers(0, bm)), g * bn - int(rng.integers(0, bn))
        else:
            M, N = int(rng.integers(1, 140)), int(rng.integers(1, 140))
        K = int(rng.integers(1, 90))
        e = int(rng.choice([1, 2, 4]))
        gm, gn = -(-M // bm), -(-N // bn)
        group = int(rng.integers(1, 6))
        caches = int(rng.choice([1, 2, 8]))
        programs = int(rng.choice([0, 1, 3, gm * gn + 2]))
        sets, ways = int(rng.choice([1, 2, 7, 64])), int(rng.choice([1, 2, 4, 16]))
        line = int(rng.choice([4, 16, 64, 128]))
        fold = (int(rng.integers(0, 8)), int(rng.choice([0, 0, 1, 3])))
        a_base = int(rng.integers(0, 5)) * 4096 + int(rng.choice([0, 2, 60]))
        b_base = a_base + M * K * e + int(rng.integers(0, 300))
        out.append((mode, M, N, K, e, (bm, bn, bk), group, caches, programs, int(rng.integers(1, 5)),
                    sets, ways, line, fold, a_base, b_base))
    return out


@pytest.mark.parametrize("case", _line_cases())
def test_line_replay_equals_oracle(case):
    (mode, M, N, K, e, block, group, caches, programs, resident, sets, ways, line, fold, a_base,
     b_base) = case
    gm, gn = -(-M // block[0]), -(-N // block[1])
    m, n = tm.tile_table(mode, gm, gn, group)
    want = l2_lines.predict_lines(m, n, M, N, K, elem_bytes=e, block=block, num_caches=caches,
                                  num_programs=programs, resident=resident, sets=sets, ways=ways,
                                  line_bytes=line, fold_from=fold[0], fold_width=fold[1],
                                  a_base=a_base, b_base=b_base)
    got = tbl.predict_l2_lines(mode, M, N, K, group, e, block, caches, programs, resident, sets, ways,
                               line, fold[0], fold[1], a_base, b_base)
    assert got[:3] == want


@pytest.mark.parametrize("name,mode,group,cluster", [
    ("group_major_g8", tm.PANEL, 8, (1, 1)),
    ("group_major_g4+remap+cluster2x2", tm.PANEL | tm.XCD_REMAP, 4, (2, 2)),
])
def test_line_replay_equals_oracle_at_8192(name, mode, group, cluster):
    # the 8192^3 persistent launch (256 programs) with the gfx950 geometry and real-looking bases
    m, n = tm.tile_table(mode, 32, 32, group, cluster=cluster)
    a_base, b_base = 0x7F1200000000, 0x7F1208200000
    want = l2_lines.predict_lines(m, n, 8192, 8192, 8192, num_programs=256, a_base=a_base,
                                  b_base=b_base, **l2_lines.GFX950)
    cl = tbl.cluster(*cluster) if cluster != (1, 1) else 0
    got = tbl.predict_l2_lines(mode | cl, 8192, 8192, 8192, group, num_programs=256, a_base=a_base,
                               b_base=b_base, **{k: v for k, v in tbl.GFX950_L2.items()})
    assert got[:3] == want


@pytest.mark.parametrize("kwargs,status", [
    (dict(mode=7), tbl.ERR_INVALID_ARG), (dict(M=0), tbl.ERR_SHAPE), (dict(K=(1 << 20) + 1), tbl.ERR_SHAPE),
    (dict(elem_bytes=3), tbl.ERR_INVALID_ARG), (dict(block=(0, 4, 4)), tbl.ERR_INVALID_ARG),
    (dict(block=(4, 4, 4097)), tbl.ERR_INVALID_ARG), (dict(num_caches=65), tbl.ERR_INVALID_ARG),
    (dict(resident=0), tbl.ERR_INVALID_ARG), (dict(sets=0), tbl.ERR_INVALID_ARG),
    (dict(ways=65), tbl.ERR_INVALID_ARG), (dict(sets=1 << 20, ways=32), tbl.ERR_INVALID_ARG),
    (dict(line_bytes=0), tbl.ERR_INVALID_ARG), (dict(fold_from=64), tbl.ERR_INVALID_ARG),
    (dict(fold_width=33), tbl.ERR_INVALID_ARG),
    (dict(a_base=(1 << 64) - 16), tbl.ERR_INVALID_ARG),
    # work bound: more than 2^33 line reads
    (dict(M=1 << 20, N=1 << 20, K=1 << 14, block=(256, 256, 32)), tbl.ERR_SHAPE),
])
def test_line_replay_invalid_arguments(kwargs, status):
    args = dict(mode=tm.ROW, M=64, N=64, K=64, group=1, elem_bytes=2, block=(16, 16, 16), num_caches=1,
                num_programs=0, resident=1, sets=4, ways=2, line_bytes=64, fold_from=0, fold_width=0,
                a_base=0, b_base=1 << 20)
    args.update(kwargs)
    with pytest.raises(tbl.TblError) as e:
        tbl.predict_l2_lines(**args)
    assert e.value.status == status


def _fixture_rows():
    rows = []
    for ln in golden_lines("l2_lines_predictions.txt"):
        t = ln.split()
        rows.append((t[0], t[1], *[int(v) for v in t[2:12]]))
    return rows


@pytest.mark.parametrize("row", _fixture_rows(), ids=lambda r: f"{r[0]}-K{r[4]}")
def test_library_reproduces_committed_line_predictions(row):
    # the fixture was written by the oracle (tests/golden/make_l2_lines_predictions.py); bench.py
    # reports the library's predictions, which must be the same numbers
    name, kind, M, N, K, mode, group, cm, cn, hits, acc, miss = row
    cl = tbl.cluster(cm, cn) if (cm, cn) != (1, 1) else 0
    got = tbl.predict_l2_lines(mode | cl, M, N, K, group, num_programs=256, **tbl.GFX950_L2)
    assert got[:3] == (hits, acc, miss)
