"""GPU parity of tbl_gemm_dynamic (the dynamic work-queue schedule) against the fp64 oracle.

What is checked:
  * values: against the oracle (full product, or sampled rows touching every tile row) to the usual
    bars (tests/_helpers.py), and bit-identical to tbl_gemm_tiled with 256x256x32 tiles (the same
    kernel arithmetic; the schedule decides only when and where a tile runs);
  * the schedule, from the trace: every order position runs exactly once, each at its (m, n) in the
    order's tile table, and every per-workgroup sequence is one that oracle.schedule's claim rules
    allow (check_dynamic_trace);
  * the workspace: launches chain on one workspace (each resets its counters), and the hand-over
    fault count stays zero;
  * edges: one workgroup running every tile, more workgroups than tiles, the minimum of nine k
    steps, ragged M, N, K, fp32 output, and queues with no local workgroup (XCD-aware with four
    workgroups), which are emptied by rotation.
Inputs come from thread_block_lds_amd.synth (A seed s, B seed s + 1).
"""

import numpy as np
import pytest
import torch

import thread_block_lds_amd as tbl
from _helpers import check_gemm, dev16, host64
from oracle import schedule as sc
from oracle import tile_maps as tm
from thread_block_lds_amd import synth

pytestmark = pytest.mark.gpu


def _run(ad, bd, mode, g, P, out_dtype=None, trace=True):
    M, N = ad.shape[0], bd.shape[1]
    T = (-(-M // 256)) * (-(-N // 256))
    Pr = P or max(1, min(T, tbl.default_num_programs(4096, 4096, 4096, persistent=True)))
    ws = tbl.dynamic_workspace(Pr)
    tr = torch.full((8 * T,), -1, dtype=torch.int32, device="cuda") if trace else None
    c = tbl.gemm_dynamic(ad, bd, mode=mode, group=g, num_programs=P, workspace=ws, out_dtype=out_dtype,
                         trace=tr)
    torch.cuda.synchronize()
    assert int(ws[9].item()) == 0, "hand-over fault"
    return c, (tr.cpu().numpy().reshape(T, 8).astype(np.int64) if trace else None)


def _check_trace(tr, mode, g, gm, gn):
    T = gm * gn
    xcd_aware = bool(mode & tm.XCD_REMAP)
    seqs = sc.check_dynamic_trace(tr[:, 0], tr[:, 1], tr[:, 4], T, xcd_aware)
    om, on = tm.tile_table(mode & ~tm.XCD_REMAP, gm, gn, g)
    assert np.array_equal(tr[:, 2], om) and np.array_equal(tr[:, 3], on)
    return seqs


@pytest.fixture(scope="module")
def square2048():
    M = N = K = 2048
    return synth.gemm_operands(M, N, K, "f16", "uniform", seed=0)


@pytest.mark.parametrize("mode,g", [(tm.ROW, 1), (tm.PANEL, 4), (tm.SERPENTINE, 2), (tm.MORTON, 1),
                                    (tm.ROW | tm.XCD_REMAP, 1), (tm.PANEL | tm.XCD_REMAP, 4),
                                    (tm.SERPENTINE | tm.XCD_REMAP, 2), (tm.XOR | tm.XCD_REMAP, 1)])
@pytest.mark.parametrize("P", [16, 64, 0])
def test_2048_orders_match_oracle_and_static(square2048, mode, g, P):
    a, b = square2048
    ad, bd = dev16(a, "f16"), dev16(b, "f16")
    c, tr = _run(ad, bd, mode, g, P)
    check_gemm(host64(c), a, b, "f16", 2048, "f16", what=f"dynamic mode {mode:#x} g{g} P{P}")
    static = tbl.gemm(ad, bd, mode=mode & ~tm.XCD_REMAP, group=g, tile=(256, 256, 32))
    torch.cuda.synchronize()
    assert torch.equal(c, static)
    seqs = _check_trace(tr, mode, g, 8, 8)
    assert sum(len(v) for v in seqs.values()) == 64


def test_workspace_chains_launches(square2048):
    a, b = square2048
    ad, bd = dev16(a, "f16"), dev16(b, "f16")
    ws = tbl.dynamic_workspace(32)
    ws[:9] = 12345                 # whatever the counters hold, each launch starts from zero
    outs = []
    for mode in (tm.PANEL, tm.PANEL | tm.XCD_REMAP, tm.SERPENTINE, tm.ROW | tm.XCD_REMAP):
        for _ in range(3):   # back to back on one stream, no synchronisation in between
            outs.append(tbl.gemm_dynamic(ad, bd, mode=mode, group=4, num_programs=32, workspace=ws))
    torch.cuda.synchronize()
    assert int(ws[9].item()) == 0
    for c in outs[1:]:
        assert torch.equal(c, outs[0])
    check_gemm(host64(outs[0]), a, b, "f16", 2048, "f16", what="chained launches")


@pytest.mark.parametrize("K", [264, 288])
def test_one_workgroup_runs_every_tile_min_k(K):
    """P = 1: one workgroup claims all 64 tiles in order; nine k steps (K = 264 with a k tail of 8,
    K = 288) are the fewest the dynamic schedule takes."""
    M, N = 2048, 2048
    a, b = synth.gemm_operands(M, N, K, "f16", "uniform", seed=5)
    for mode in (tm.PANEL, tm.PANEL | tm.XCD_REMAP):
        c, tr = _run(dev16(a, "f16"), dev16(b, "f16"), mode, 4, 1)
        check_gemm(host64(c), a, b, "f16", K, "f16", what=f"P=1 mode {mode:#x}")
        seqs = _check_trace(tr, mode, 4, 8, 8)
        assert len(seqs) == 1
        p = next(iter(seqs))
        if mode & tm.XCD_REMAP:   # own block first, then the others in rotation
            x = int(tr[0, 4])
            blocks = sc.queue_blocks(64, True)
            want = [t for q in range(8) for t in range(*blocks[(x + q) % 8])]
            assert seqs[p] == want
        else:
            assert seqs[p] == list(range(64))


def test_more_workgroups_than_tiles():
    M, N, K = 1024, 768, 512      # 4 x 3 = 12 tiles, 64 workgroups
    a, b = synth.gemm_operands(M, N, K, "f16", "uniform", seed=6)
    for mode in (tm.ROW, tm.ROW | tm.XCD_REMAP):
        c, tr = _run(dev16(a, "f16"), dev16(b, "f16"), mode, 1, 64)
        check_gemm(host64(c), a, b, "f16", K, "f16", what=f"P > T mode {mode:#x}")
        _check_trace(tr, mode, 1, 4, 3)


@pytest.mark.parametrize("mode", [tm.PANEL, tm.PANEL | tm.XCD_REMAP])
def test_more_workgroups_than_resident(mode):
    """1024 and 777 workgroups on 256 tiles: the first 256 take their first-round tiles, the rest
    (dispatched as earlier ones finish) find every queue empty and leave."""
    M, N, K = 4096, 4096, 512
    a, b = synth.gemm_operands(M, N, K, "f16", "uniform", seed=9)
    ad, bd = dev16(a, "f16"), dev16(b, "f16")
    static = tbl.gemm(ad, bd, mode=mode & ~tm.XCD_REMAP, group=4, tile=(256, 256, 32))
    rows = np.arange(3, M, 97)
    for P in (1024, 777):
        c, tr = _run(ad, bd, mode, 4, P)
        assert torch.equal(c, static), P
        check_gemm(host64(c)[rows], a, b, "f16", K, "f16", rows, what=f"P={P} mode {mode:#x}")
        seqs = _check_trace(tr, mode, 4, 16, 16)
        assert max(seqs) < 256 and all(len(v) == 1 for v in seqs.values())


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_ragged_fp32_out(dtype):
    M, N, K = 1000, 776, 1000     # partial tiles at M and N edges, a k tail of 8
    a, b = synth.gemm_operands(M, N, K, dtype, "uniform" if dtype == "f16" else "normal", seed=7)
    ad, bd = dev16(a, dtype), dev16(b, dtype)
    c, tr = _run(ad, bd, tm.SERPENTINE | tm.XCD_REMAP, 2, 3, out_dtype=torch.float32)
    check_gemm(host64(c), a, b, dtype, K, "f32", what=f"ragged {dtype} fp32 out")
    _check_trace(tr, tm.SERPENTINE | tm.XCD_REMAP, 2, 4, 4)
    static = tbl.gemm(ad, bd, mode=tm.SERPENTINE, group=2, out_dtype=torch.float32, tile=(256, 256, 32))
    torch.cuda.synchronize()
    assert torch.equal(c, static)


def test_queues_without_local_workgroups_are_stolen():
    """Four workgroups, XCD-aware: the blocks of XCDs with no workgroup are emptied by rotation."""
    M, N, K = 4096, 2048, 288     # 16 x 8 = 128 tiles, 16 per block
    a, b = synth.gemm_operands(M, N, K, "f16", "uniform", seed=8)
    ad, bd = dev16(a, "f16"), dev16(b, "f16")
    c, tr = _run(ad, bd, tm.ROW | tm.XCD_REMAP, 1, 4)
    seqs = _check_trace(tr, tm.ROW | tm.XCD_REMAP, 1, 16, 8)
    xcds = {int(tr[seqs[p][0], 4]) for p in seqs}
    blocks = sc.queue_blocks(128, True)
    run_on = np.array([tr[t, 4] for t in range(128)])
    empty = [x for x in range(8) if x not in xcds]
    for x in empty:                # every tile of an unserved block ran on another XCD
        assert np.all(run_on[blocks[x][0]:blocks[x][1]] != x)
    rows = np.arange(0, M, 61)
    check_gemm(host64(c)[rows], a, b, "f16", K, "f16", rows, what="stolen blocks")


def test_c3_8192_bf16_xcd_aware_equals_static_remap():
    """8192^3 bf16 N(0,1)/sqrt(K), persistent: serpentine 8 and group-major 8 with per-XCD queues
    give the bits of the static schedule with the remap; sampled rows against the oracle."""
    M = N = K = 8192
    a, b = synth.gemm_operands(M, N, K, "bf16", "normal", seed=0)
    ad, bd = dev16(a, "bf16"), dev16(b, "bf16")
    rows = np.array(sorted({r * 256 + (r * 37) % 256 for r in range(32)}))
    static = tbl.gemm(ad, bd, mode=tm.SERPENTINE | tm.XCD_REMAP, group=8, persistent=True)
    for mode in (tm.SERPENTINE | tm.XCD_REMAP, tm.PANEL | tm.XCD_REMAP, tm.PANEL):
        c, tr = _run(ad, bd, mode, 8, 0)
        assert torch.equal(c, static), mode
        check_gemm(host64(c[torch.from_numpy(rows).cuda()]), a, b, "bf16", K, "bf16", rows,
                   what=f"8192^3 dynamic {mode:#x}")
        _check_trace(tr, mode, 8, 32, 32)
        del c


def test_c4_rectangular_partial_groups():
    """10240 x 6144 x 2048 fp16 (40 x 24 tiles, 960 over 256 workgroups): panel g16 (groups of 16,
    16 and 8 rows) and serpentine s16 (a last strip of 8 columns), one queue and a queue per XCD
    (blocks of 120 positions); bits of the static schedule, sampled rows against the oracle."""
    M, N, K = 10240, 6144, 2048
    a, b = synth.gemm_operands(M, N, K, "f16", "uniform", seed=0)
    ad, bd = dev16(a, "f16"), dev16(b, "f16")
    rows = np.array(sorted({r * 256 + (r * 53) % 256 for r in range(40)}))
    static = tbl.gemm(ad, bd, mode=tm.PANEL, group=16, persistent=True)
    for mode, g in ((tm.PANEL, 16), (tm.PANEL | tm.XCD_REMAP, 16), (tm.SERPENTINE, 16),
                    (tm.SERPENTINE | tm.XCD_REMAP, 16)):
        c, tr = _run(ad, bd, mode, g, 0)
        assert torch.equal(c, static), mode
        check_gemm(host64(c[torch.from_numpy(rows).cuda()]), a, b, "f16", K, "f16", rows,
                   what=f"C4 dynamic {mode:#x} g{g}")
        _check_trace(tr, mode, g, 40, 24)


def test_binding_checks_workspace():
    a = torch.zeros((512, 512), dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        tbl.gemm_dynamic(a, a, num_programs=4, workspace=torch.zeros(1024, dtype=torch.int32))
    with pytest.raises(TypeError):
        tbl.gemm_dynamic(a, a, num_programs=4,
                         workspace=torch.zeros(1024, dtype=torch.int64, device="cuda"))
    with pytest.raises(tbl.TblError) as e:
        tbl.gemm_dynamic(a, a, num_programs=4, workspace=torch.zeros(64, dtype=torch.int32, device="cuda"))
    assert e.value.status == tbl.ERR_INVALID_ARG
    small_k = torch.zeros((512, 192), dtype=torch.float16, device="cuda")
    with pytest.raises(tbl.TblError) as e:
        tbl.gemm_dynamic(small_k, torch.zeros((192, 512), dtype=torch.float16, device="cuda"),
                         num_programs=4, workspace=tbl.dynamic_workspace(4))
    assert e.value.status == tbl.ERR_SHAPE
