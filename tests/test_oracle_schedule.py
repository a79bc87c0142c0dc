"""Pins of the dynamic-schedule oracle (oracle/schedule.py) to the pages and to scheduling theory.

* Equal tile times: claims arrive in program order, so the dynamic schedule hands out exactly the
  stride schedule of the pages ([P1] "Persistent vs. non-persistent launch"; [P3] "Example 1"'s
  printed work lists), and its XCD-aware form hands out the XCD-remapped stride schedule.
* Unequal tile times: hand-worked cases, Graham's bound for greedy list scheduling (lookahead 0:
  makespan <= sum/P + (1 - 1/P) max), brute-force optima on tiny instances, and the bound
  makespan <= sum/P + 2 max for one-ahead claims (proof in test_lookahead_one_bound).
"""

import itertools

import numpy as np
import pytest

from oracle import schedule as sc
from oracle import tile_maps as tm
from conftest import golden_sections


@pytest.mark.parametrize("P,T", [(1, 5), (3, 16), (4, 4), (7, 30), (16, 16), (256, 1024), (256, 960),
                                 (5, 3)])
@pytest.mark.parametrize("lookahead", [0, 1])
def test_equal_times_give_the_stride_schedule(P, T, lookahead):
    tiles, start, _, owner, makespan = sc.simulate_dynamic([1.0] * T, P, lookahead=lookahead)
    for p in range(P):
        assert tiles[p] == sc.stride_tiles(p, P, T)
    assert makespan == -(-T // P)
    assert np.all(owner >= 0)


def test_p3_example1_work_lists():
    """[P3] Example 1: 4x4 tiles, 3 clusters; the printed per-cluster work_idx lists."""
    sec = golden_sections("p3_example1_clusters.txt")
    tiles, *_ = sc.simulate_dynamic([1.0] * 16, 3, lookahead=1)
    for ln in sec["work"][1]:
        c, _, ids = ln.partition(":")
        assert tiles[int(c)] == [int(v) for v in ids.split()]


@pytest.mark.parametrize("P,T", [(8, 64), (16, 64), (256, 1024), (256, 256), (64, 960), (8, 8)])
def test_xcd_aware_equal_times_give_the_remapped_stride_schedule(P, T):
    """Programs on XCD x = p mod 8 split block x in program order: position = remap(p + i P)."""
    tiles, *_ = sc.simulate_dynamic([1.0] * T, P, lookahead=1, xcd_aware=True)
    for p in range(P):
        want = [int(tm.xcd_remap(t, T)) for t in sc.stride_tiles(p, P, T)]
        assert tiles[p] == want


def test_queue_blocks_partition():
    for T in [0, 1, 5, 7, 8, 9, 63, 64, 960, 1000]:
        blocks = sc.queue_blocks(T, True)
        assert blocks[0][0] == 0 and blocks[-1][1] == T and len(blocks) == 8
        assert all(blocks[i][1] == blocks[i + 1][0] for i in range(7))
        sizes = [hi - lo for lo, hi in blocks]
        assert max(sizes) - min(sizes) <= 1
    assert sc.queue_blocks(10, False) == [(0, 10)]


def test_hand_worked_case():
    """Two programs, tiles taking 3, 1, 1. Claiming on finishing: program 1 runs tiles 1 and 2
    (done at 3). Claiming one ahead: program 0 claims tile 2 when it starts tile 0, as the stride
    schedule would (done at 4) -- the price of hiding the claim behind a tile."""
    tiles, start, finish, owner, ms = sc.simulate_dynamic([3, 1, 1], 2, lookahead=0)
    assert tiles == [[0], [1, 2]] and ms == 3.0
    assert start.tolist() == [0.0, 0.0, 1.0]
    tiles, start, finish, owner, ms = sc.simulate_dynamic([3, 1, 1], 2, lookahead=1)
    assert tiles == [[0, 2], [1]] and ms == 4.0
    assert finish.tolist() == [3.0, 1.0, 4.0]


def test_slow_program_is_balanced():
    """Tiles 0, 4, 8, ... take 5 units, the rest 1 (program 0's stride share is slow): the static
    stride schedule ends at 5 * 8 = 40; claiming balances it."""
    T, P = 32, 4
    d = [5.0 if t % 4 == 0 else 1.0 for t in range(T)]
    static = max(sum(d[t] for t in sc.stride_tiles(p, P, T)) for p in range(P))
    assert static == 40.0
    for la in (0, 1):
        *_, ms = sc.simulate_dynamic(d, P, lookahead=la)
        assert ms <= sum(d) / P + 2 * max(d) and ms < static


def _brute_force_optimum(d, P):
    best = float("inf")
    for assign in itertools.product(range(P), repeat=len(d)):
        loads = [0.0] * P
        for t, p in enumerate(assign):
            loads[p] += d[t]
        best = min(best, max(loads))
    return best


@pytest.mark.parametrize("seed", range(12))
def test_graham_bound_and_optimum(seed):
    rng = np.random.default_rng(seed)
    P = int(rng.integers(2, 4))
    T = int(rng.integers(1, 8))
    d = rng.integers(1, 10, size=T).astype(float).tolist()
    *_, ms = sc.simulate_dynamic(d, P, lookahead=0)
    assert ms <= sum(d) / P + (1 - 1 / P) * max(d) + 1e-9
    opt = _brute_force_optimum(d, P)
    assert opt - 1e-9 <= ms <= (2 - 1 / P) * opt + 1e-9


@pytest.mark.parametrize("seed", range(20))
@pytest.mark.parametrize("xcd_aware", [False, True])
def test_lookahead_one_bound(seed, xcd_aware):
    """No program idles before the last successful claim (it idles only after a claim failed, and
    every claim fails only after all succeeded), so P * c <= sum for that claim's time c; a claim made
    at c is for a tile that starts when the claimer's current tile (started at c) ends, so every tile
    ends by c + 2 max. Hence makespan <= sum/P + 2 max; each position runs once."""
    rng = np.random.default_rng(100 + seed)
    P = int(rng.integers(1, 40))
    T = int(rng.integers(0, 300))
    d = rng.exponential(1.0, size=T).tolist()
    tiles, start, finish, owner, ms = sc.simulate_dynamic(d, P, lookahead=1, xcd_aware=xcd_aware)
    assert sorted(t for ts in tiles for t in ts) == list(range(T))
    if T:
        assert ms <= sum(d) / P + 2 * max(d) + 1e-9
        # a program's tiles run back to back from time 0 in the order it claimed them
        for p in range(P):
            if tiles[p]:
                s = start[tiles[p]]
                f = finish[tiles[p]]
                assert s[0] == 0.0 and np.allclose(s[1:], f[:-1])
    program = owner
    iteration = np.zeros(T, dtype=np.int64)
    for p in range(P):
        for i, t in enumerate(tiles[p]):
            iteration[t] = i
    xcd = np.array([p % 8 for p in program], dtype=np.int64)
    sc.check_dynamic_trace(program, iteration, xcd, T, xcd_aware)


def test_steal_takes_the_fullest_block():
    """Hand case, T = 16 (blocks of 2), four programs on XCDs 0..3, program 0's tiles 10x slower:
    programs 1..3 empty their blocks, then each steals from the block with the most positions left
    (4..7 hold 2 each; ties go to the nearest block after the thief's own XCD)."""
    d = [1.0] * 16
    d[0] = d[1] = 10.0
    tiles, _, _, owner, ms = sc.simulate_dynamic(d, 4, lookahead=1, xcd_aware=True)
    assert tiles[0][:2] == [0, 1]
    assert tiles[1][:2] == [2, 3] and tiles[2][:2] == [4, 5] and tiles[3][:2] == [6, 7]
    # time 0, second claims (one ahead): 0 -> 1, 1 -> 3, 2 -> 5, 3 -> 7, all from their own blocks.
    # time 1, programs 1..3 claim again and find their blocks empty. Program 1: blocks 4..7 have 2
    # left each, the nearest after XCD 1 is block 4 -> position 8. Program 2: block 4 now has 1, 5..7
    # have 2, nearest is 5 -> 10. Program 3: 6 and 7 have 2, nearest is 6 -> 12.
    assert tiles[1][2] == 8 and tiles[2][2] == 10 and tiles[3][2] == 12
    assert ms <= sum(d) / 4 + 2 * max(d)


def test_xcd_aware_steals_from_other_blocks():
    """Equal times: every position stays on its block's XCD. Block 0's tiles taking 3 units and the
    rest 1: the other XCDs' programs empty their own blocks, then take block 0's remaining ones."""
    T, P = 256, 32
    xcd_of = lambda p: p % 8
    tiles, _, _, owner, ms = sc.simulate_dynamic(
        [1.0] * T, P, lookahead=1, xcd_aware=True, xcd_of=xcd_of)
    assert all(owner[t] % 8 == t // 32 for t in range(T))          # equal times: no stealing
    slow = [3.0 if (t // 32) == 0 else 1.0 for t in range(T)]
    tiles, _, _, owner, ms = sc.simulate_dynamic(slow, P, lookahead=1, xcd_aware=True, xcd_of=xcd_of)
    stolen = [t for t in range(32) if owner[t] % 8 != 0]
    assert stolen and all(owner[t] % 8 != 0 for t in stolen)
    assert ms < 3.0 * 8     # without stealing, XCD 0's four programs run 8 slow tiles each


def _trace_from(tiles, T):
    program = np.full(T, -1, dtype=np.int64)
    iteration = np.full(T, -1, dtype=np.int64)
    for p, ts in enumerate(tiles):
        for i, t in enumerate(ts):
            program[t] = p
            iteration[t] = i
    return program, iteration


def test_trace_checker_rejects_planted_mistakes():
    T, P = 64, 16
    tiles, *_ = sc.simulate_dynamic([1.0] * T, P, lookahead=1, xcd_aware=True)
    program, iteration = _trace_from(tiles, T)
    xcd = program % 8
    sc.check_dynamic_trace(program, iteration, xcd, T, True)
    bad = program.copy()
    bad[5] = -1                                        # a position never ran
    with pytest.raises(AssertionError):
        sc.check_dynamic_trace(bad, iteration, xcd, T, True)
    it2 = iteration.copy()
    it2[tiles[0][1]] = 0                               # two tiles with one iteration index
    with pytest.raises(AssertionError):
        sc.check_dynamic_trace(program, it2, xcd, T, True)
    it3 = iteration.copy()                             # program 0 runs its tiles in reverse
    for i, t in enumerate(reversed(tiles[0])):
        it3[t] = i
    with pytest.raises(AssertionError):
        sc.check_dynamic_trace(program, it3, xcd, T, True)
    x2 = xcd.copy()
    x2[tiles[0][0]] = 3                                # one program on two XCDs
    with pytest.raises(AssertionError):
        sc.check_dynamic_trace(program, iteration, x2, T, True)
    p2 = program.copy()                                # program 0 (XCD 0) also runs a block-7 tile
    it4 = iteration.copy()
    x4 = xcd.copy()
    t7 = tiles[7][-1]                                  # its last, so program 7 stays consistent
    p2[t7], it4[t7], x4[t7] = 0, len(tiles[0]), 0
    sc.check_dynamic_trace(p2, it4, x4, T, True)       # block 7 comes after block 0 in XCD 0's rotation...
    it4[t7] = 0                                        # ...but not before it
    for i, t in enumerate(tiles[0]):
        it4[t] = i + 1
    with pytest.raises(AssertionError):
        sc.check_dynamic_trace(p2, it4, x4, T, True)
    # the single-queue form demands increasing positions per program
    tiles1, *_ = sc.simulate_dynamic([1.0] * T, P, lookahead=1)
    program1, iteration1 = _trace_from(tiles1, T)
    sc.check_dynamic_trace(program1, iteration1, program1 % 8, T, False)
    it5 = iteration1.copy()
    a, b = tiles1[2][0], tiles1[2][1]
    it5[a], it5[b] = it5[b], it5[a]
    with pytest.raises(AssertionError):
        sc.check_dynamic_trace(program1, it5, program1 % 8, T, False)
