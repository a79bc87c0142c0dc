"""Oracle: persistent schedules -- the static stride schedule and a dynamic (work-queue) schedule.

TEST INFRASTRUCTURE (see the package docstring): not imported by the library.

Sources:
  [P1] "CUDA Thread Block Swizzle" (leimao.github.io), section "CUDA Thread Block Swizzle
       Benchmark", the benchmark's notes "Persistent vs. non-persistent launch" (a persistent
       program p visits tile ids p, p + P, p + 2P, ...) and "Known limitations" (that assignment is
       static: no counter hands out tiles at run time, so nothing balances the programs' loads).
  [P3] "tvm_tirx ... ClusterPersistentScheduler2D" (tvm.apache.org), "Example 1: Basic persistent
       kernel" (the per-cluster work lists of the stride schedule).

The dynamic schedule is the counterpart that [P1] names but does not define. READINGS, the plainest
ones its notes support:
  * One shared counter hands out the positions 0, 1, 2, ... of the tile order in increasing order;
    a program takes the next one whenever it needs a tile; a position >= T means no work is left
    and the program stops.
  * Claims run one tile ahead (lookahead 1): a program claims its first tile when it starts and its
    (j+1)-th tile when it starts its j-th, so the claim's latency hides behind a tile of work.
    Lookahead 0 (claim on finishing a tile) is the textbook greedy list schedule.
  * XCD-aware variant (gfx950 has eight XCDs with private L2s): the order's positions are cut into
    X contiguous blocks, block x = [floor(x T / X), floor((x + 1) T / X)), each with its own counter.
    A program on XCD x claims from block x while it has positions left; then from the block with
    the most unclaimed positions (ties: the nearest after x in the order x + 1, x + 2, ... mod X),
    keeping to that block while it lasts; it stops when every block is empty.
  * Simultaneous claims are served in order of claim number, then program index (in the kernel they
    race; the tests of GPU traces check only what holds for every interleaving).
"""

import heapq
from collections import deque

import numpy as np


def stride_tiles(p, P, T):
    """[P1] persistent loop; [P3] Example 1: program p visits ids p, p + P, p + 2P, ... < T."""
    return list(range(p, T, P))


def queue_blocks(T, xcd_aware, X=8):
    """Position ranges [lo, hi) of the work queues: one queue [0, T), or X contiguous blocks."""
    if not xcd_aware:
        return [(0, T)]
    return [(x * T // X, (x + 1) * T // X) for x in range(X)]


class _Queues:
    """The claim counters of one launch; claim() follows the READINGS in the module docstring."""

    def __init__(self, T, xcd_aware, X):
        self.blocks = queue_blocks(T, xcd_aware, X)
        self.count = [0] * len(self.blocks)
        self.xcd_aware = xcd_aware
        self.X = X

    def left(self, q):
        lo, hi = self.blocks[q]
        return max(0, hi - lo - self.count[q])

    def claim(self, cursor):
        """cursor = [own queue, queue now claimed from]; returns a position or -1."""
        q = cursor[1]
        lo, hi = self.blocks[q]
        c = self.count[q]
        self.count[q] += 1
        if lo + c < hi:
            return lo + c
        if not self.xcd_aware:
            return -1
        own = cursor[0]
        best = max(range(self.X), key=lambda r: (self.left(r), -((r - own) % self.X)))
        if self.left(best) == 0:
            return -1
        cursor[1] = best
        lo, hi = self.blocks[best]
        c = self.count[best]
        self.count[best] += 1
        return lo + c


def simulate_dynamic(durations, P, lookahead=1, xcd_aware=False, xcd_of=None, X=8):
    """Event simulation of the dynamic schedule.

    durations: per order position, the time its tile takes (T = len(durations)).
    P: programs, all starting at time 0. xcd_of(p): the XCD of program p (default p mod X).
    Events at one time: tile ends first (by program), then claims by claim number, then program.
    Returns (tiles, start, finish, owner, makespan): tiles[p] = positions in the order p ran them;
    start, finish and owner are indexed by position.
    """
    durations = [float(d) for d in durations]
    T = len(durations)
    if P < 1 or lookahead not in (0, 1):
        raise ValueError("P >= 1 and lookahead 0 or 1")
    xcd_of = xcd_of or (lambda p: p % X)
    queues = _Queues(T, xcd_aware, X)
    cursors = [[xcd_of(p) % X] * 2 if xcd_aware else [0, 0] for p in range(P)]
    tiles = [[] for _ in range(P)]
    start = np.full(T, np.nan)
    finish = np.full(T, np.nan)
    owner = np.full(T, -1, dtype=np.int64)
    pending = [deque() for _ in range(P)]   # claimed, not started
    running = [False] * P
    done = [False] * P                      # a claim found no work left
    claims = [0] * P
    END = -1                                # event key of a tile end
    events = [(0.0, 0, p) for p in range(P)]
    heapq.heapify(events)

    def begin(p, now):
        pos = pending[p].popleft()
        start[pos] = now
        finish[pos] = now + durations[pos]
        owner[pos] = p
        tiles[p].append(pos)
        running[p] = True
        heapq.heappush(events, (finish[pos], END, p))
        if lookahead == 1 and not done[p]:
            heapq.heappush(events, (now, claims[p], p))   # the next tile's claim

    while events:
        now, key, p = heapq.heappop(events)
        if key == END:
            running[p] = False
            if pending[p]:
                begin(p, now)
            elif lookahead == 0 and not done[p]:
                heapq.heappush(events, (now, claims[p], p))
            continue
        pos = queues.claim(cursors[p])
        claims[p] += 1
        if pos < 0:
            done[p] = True
            continue
        pending[p].append(pos)
        if not running[p]:
            begin(p, now)
    makespan = float(np.max(finish)) if T else 0.0
    return tiles, start, finish, owner, makespan


def check_dynamic_trace(program, iteration, xcd, T, xcd_aware, X=8):
    """What every run of the dynamic schedule satisfies, whatever the order of racing claims.

    program, iteration, xcd: per order position, the program that ran it, its index among that
    program's tiles, and the XCD that program ran on. Raises AssertionError on a violation;
    returns {program: positions in iteration order}.
    """
    program = np.asarray(program)
    iteration = np.asarray(iteration)
    xcd = np.asarray(xcd)
    assert program.shape == (T,) and iteration.shape == (T,) and xcd.shape == (T,)
    assert np.all(program >= 0), "a position was never run"
    blocks = queue_blocks(T, xcd_aware, X)
    block_of = np.empty(T, dtype=np.int64)
    for q, (lo, hi) in enumerate(blocks):
        block_of[lo:hi] = q
    seqs = {}
    for p in np.unique(program):
        pos = np.flatnonzero(program == p)
        order = np.argsort(iteration[pos], kind="stable")
        pos = pos[order]
        it = iteration[pos]
        assert np.array_equal(it, np.arange(len(pos))), f"program {p}: iterations {it.tolist()}"
        xs = np.unique(xcd[pos])
        assert len(xs) == 1, f"program {p} ran on XCDs {xs.tolist()}"
        if not xcd_aware:
            assert np.all(np.diff(pos) > 0), f"program {p}: claims not increasing {pos.tolist()}"
        else:
            own = int(xs[0])
            mine = block_of[pos] == own
            n_own = int(np.sum(mine))
            assert np.all(mine[:n_own]), f"program {p}: left its own block and came back {pos.tolist()}"
            for q in np.unique(block_of[pos]):
                sel = pos[block_of[pos] == q]
                assert np.all(np.diff(sel) > 0), f"program {p}: claims in block {q} not increasing"
        seqs[int(p)] = pos.tolist()
    return seqs
