"""GPU test: the library's launches captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.
Every entry point enqueues kernels only (the dynamic schedule zeroes its counters with a kernel,
never a memset) and allocates nothing when its outputs are given, so a serving loop can capture it.
The graph is replayed several times with eager work and synchronisations in between, and every
replay must give the eager results bit for bit: the fast GEMM kernels (persistent, remapped
panel order), the general path (N and K not multiples of 8), the allocation-free dynamic schedule,
a transpose and a tile table."""

import numpy as np
import pytest
import torch

import thread_block_lds_amd as tbl
from oracle import tile_maps as tm
from thread_block_lds_amd import synth

from _helpers import dev16

pytestmark = pytest.mark.gpu


def test_captured_launches_replay_bit_identical():
    a, b = synth.gemm_operands(1024, 1024, 512, "f16", "uniform", seed=21)
    ad, bd = dev16(a, "f16"), dev16(b, "f16")
    oa, ob = synth.gemm_operands(300, 263, 77, "bf16", "normal", seed=22)
    oad, obd = dev16(oa, "bf16"), dev16(ob, "bf16")
    da, db = synth.gemm_operands(600, 520, 384, "f16", "uniform", seed=23)
    dad, dbd = dev16(da, "f16"), dev16(db, "f16")
    x = torch.from_numpy(synth.i32_uniform((1024, 2048), 24)).cuda()
    P = 64

    def launch(outs):
        tbl.gemm(ad, bd, c=outs[0], mode=tm.PANEL | tm.XCD_REMAP, group=4, persistent=True, num_programs=P)
        tbl.gemm(oad, obd, c=outs[1], mode=tm.SERPENTINE, group=2)
        tbl.gemm_dynamic_noalloc(dad, dbd, c=outs[2], mode=tm.PANEL | tm.XCD_REMAP, group=2, num_programs=P)
        tbl.transpose_i32(x, out=outs[3], layout=tbl.T_XOR)
        tbl.tile_map(tm.SERPENTINE, 40, 24, 3, out_m=outs[4], out_n=outs[5])

    def fresh():
        return [torch.empty((1024, 1024), dtype=torch.float16, device="cuda"),
                torch.empty((300, 263), dtype=torch.bfloat16, device="cuda"),
                torch.empty((600, 520), dtype=torch.float16, device="cuda"),
                torch.empty((2048, 1024), dtype=torch.int32, device="cuda"),
                torch.empty(960, dtype=torch.int32, device="cuda"),
                torch.empty(960, dtype=torch.int32, device="cuda")]

    eager = fresh()
    launch(eager)
    torch.cuda.synchronize()
    om, on = tm.tile_table(tm.SERPENTINE, 40, 24, 3)
    assert np.array_equal(eager[4].cpu().numpy(), om) and np.array_equal(eager[5].cpu().numpy(), on)
    assert np.array_equal(eager[3].cpu().numpy(), x.cpu().numpy().T)

    static = fresh()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up on a side stream, as capture wants
        launch(static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch(static)
    torch.cuda.synchronize()

    for r in range(4):
        for t in static:   # poison the outputs eagerly, so each replay must write them again
            if t.dtype == torch.int32:
                t.fill_(-7)
            else:
                t.fill_(float("nan"))
        # eager library work between the replays, on the default stream
        tbl.gemm(oad, obd, mode=tm.ROW, persistent=True)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (got, want) in enumerate(zip(static, eager)):
            assert torch.equal(got.view(torch.int16) if got.dtype != torch.int32 else got,
                               want.view(torch.int16) if want.dtype != torch.int32 else want), (r, i)
