"""GPU tests of the degenerate shapes, through the binding and the C ABI: empty outputs (M = 0 or
N = 0) enqueue nothing; K = 0 sets every element of C to +0, the empty sum of the product "CUDA
Thread Block Swizzle" (section "CUDA Thread Block Swizzle Benchmark") computes, equal to the
oracle's; empty transposes and tile tables. The K = 0 fill is checked bit for bit (+0, not -0),
at ragged byte counts (a tail shorter than 16 bytes) and for bytes past C left untouched."""

import numpy as np
import pytest
import torch

import thread_block_lds_amd as tbl
from oracle import gemm as og
from oracle import tile_maps as tm
from oracle.transpose import transpose_i32
from thread_block_lds_amd import synth

pytestmark = pytest.mark.gpu

DT = {"f16": torch.float16, "bf16": torch.bfloat16}


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("f32_out", [False, True])
@pytest.mark.parametrize("M,N", [(1, 1), (77, 9), (300, 136), (1000, 1001), (4096, 4096)])
def test_k0_fills_zero_and_nothing_past_c(dtype, f32_out, M, N):
    out = torch.float32 if f32_out else DT[dtype]
    a = torch.empty((M, 0), dtype=DT[dtype], device="cuda")
    b = torch.empty((0, N), dtype=DT[dtype], device="cuda")
    # C is the front of a larger buffer whose every byte starts as 0xFF (a NaN in each type)
    esize = 4 if f32_out else 2
    spare = 64
    raw = torch.full((M * N * esize + spare,), 0xFF, dtype=torch.uint8, device="cuda")
    c = raw[: M * N * esize].view(out).view(M, N)
    tbl.gemm(a, b, c=c, mode=tm.PANEL, group=4)
    torch.cuda.synchronize()
    host = raw.cpu().numpy()
    assert not host[: M * N * esize].any(), "every byte of C is zero (+0 in every output type)"
    assert (host[M * N * esize:] == 0xFF).all(), "bytes past C untouched"
    ref = og.gemm(np.zeros((M, 0), np.uint16), np.zeros((0, N), np.uint16), dtype)
    assert ref.shape == (M, N) and np.array_equal(c.double().cpu().numpy(), ref)


@pytest.mark.parametrize("tile", [(64, 64, 32), (128, 128, 32), (256, 256, 32)])
def test_k0_tiled_leaves_trace_and_matches_tbl_gemm(tile):
    M, N = 520, 264
    a = torch.empty((M, 0), dtype=torch.float16, device="cuda")
    b = torch.empty((0, N), dtype=torch.float16, device="cuda")
    T = -(-M // tile[0]) * -(-N // tile[1])
    trace = torch.full((8 * T,), -7, dtype=torch.int32, device="cuda")
    c = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    tbl.gemm(a, b, c=c, tile=tile, trace=trace, mode=tm.SERPENTINE | tm.XCD_REMAP, group=2, persistent=True)
    torch.cuda.synchronize()
    assert (c.view(torch.int16) == 0).all()
    assert (trace == -7).all(), "no tile runs for K = 0"


@pytest.mark.parametrize("M,N,K", [(0, 512, 512), (512, 0, 512), (0, 0, 0), (0, 9, 77), (33, 0, 0)])
def test_empty_output_enqueues_nothing(M, N, K):
    a = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    b = torch.randn((K, N), device="cuda").to(torch.bfloat16)
    for persistent in (False, True):
        c = tbl.gemm(a, b, persistent=persistent)
        assert c.shape == (M, N) and c.dtype == torch.bfloat16
        c = tbl.gemm(a, b, out_dtype=torch.float32, tile=(128, 128, 32),
                     trace=torch.empty(0, dtype=torch.int32, device="cuda"))
        assert c.shape == (M, N) and c.dtype == torch.float32
    torch.cuda.synchronize()


def test_k0_then_normal_gemm_on_the_same_c():
    # the fill leaves C as the oracle's zeros, and an ordinary GEMM into the same C afterwards
    # overwrites it completely
    M, N, K = 300, 136, 520
    c = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    z = torch.empty((M, 0), dtype=torch.float16, device="cuda")
    tbl.gemm(z, torch.empty((0, N), dtype=torch.float16, device="cuda"), c=c)
    torch.cuda.synchronize()
    assert (c == 0).all()
    a = synth.int_valued((M, K), 3, -2, 2, "f16")
    b = synth.int_valued((K, N), 4, -2, 2, "f16")
    ad = torch.from_numpy(a.view(np.int16)).view(torch.float16).cuda()
    bd = torch.from_numpy(b.view(np.int16)).view(torch.float16).cuda()
    tbl.gemm(ad, bd, c=c)
    torch.cuda.synchronize()
    assert np.array_equal(c.double().cpu().numpy(), og.gemm(a, b, "f16"))


def test_empty_transpose_tile_map_and_copy():
    for rows, cols in [(0, 64), (128, 0), (0, 0)]:
        x = torch.empty((rows, cols), dtype=torch.int32, device="cuda")
        for layout in (tbl.T_NAIVE, tbl.T_PADDED, tbl.T_XOR):
            y = tbl.transpose_i32(x, layout=layout)
            assert y.shape == (cols, rows)
            assert np.array_equal(y.cpu().numpy(), transpose_i32(x.cpu().numpy()))
    for gm, gn in [(0, 8), (8, 0), (0, 0)]:
        m, n, st = tbl.tile_map(tm.SERPENTINE, gm, gn, 2)
        assert st == tbl.OK and m.numel() == 0 and n.numel() == 0
        om, on = tm.tile_table(tm.SERPENTINE, gm, gn, 2)
        assert len(om) == 0 and len(on) == 0
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    assert tbl.copy16(e).numel() == 0
    # a non-empty call after the empty ones still works
    x = torch.from_numpy(synth.i32_uniform((64, 128), 1)).cuda()
    assert np.array_equal(tbl.transpose_i32(x).cpu().numpy(), x.cpu().numpy().T)
    torch.cuda.synchronize()
