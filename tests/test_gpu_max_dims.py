"""GPU parity at the library's largest accepted dimension, 2^20 (the C-ABI returns TBL_ERR_SHAPE
above it), one axis at a time, so that every address the kernels form spans the widest range they
accept: a 2^20-deep k loop, 2^20 rows of A and C, 2^20 columns of B and C, and a 2^20-row or
2^20-column transpose.

The GEMMs run on integer inputs in [-2, 2] with fp32 output: every partial sum is an integer of
magnitude at most 4 K = 2^22 < 2^24, so fp32 holds it exactly and the result must equal the fp64
oracle of "CUDA Thread Block Swizzle" (section "CUDA Thread Block Swizzle Benchmark", the GEMM its
tiles compute) bit for bit. The transposes follow "CUDA Swizzle & bank conflict" (section "Case
Study / Matrix Transpose") and are bit-exact in all three LDS layouts."""

import numpy as np
import pytest
import torch

import thread_block_lds_amd as tbl
from oracle import gemm as og
from oracle import tile_maps as tm
from oracle.transpose import transpose_i32 as oracle_transpose
from thread_block_lds_amd import synth

from _helpers import check_gemm, dev16, host64

pytestmark = pytest.mark.gpu

BIG = 1 << 20


def _ints(M, N, K, seed):
    a = synth.int_valued((M, K), seed, -2, 2, "bf16")
    b = synth.int_valued((K, N), seed + 1, -2, 2, "bf16")
    return a, b


def test_max_k_every_tile_size():
    # one output tile, 32768 k steps, in each kernel; 16-bit output as well (bf16 of an integer
    # up to 2^22 rounds, so it is checked against the bars instead)
    M = N = 64
    a, b = _ints(M, N, BIG, 71)
    ad, bd = dev16(a, "bf16"), dev16(b, "bf16")
    ref = og.gemm_rows(a, b, "bf16", np.arange(M))
    assert np.max(np.abs(ref)) < 2 ** 24
    for tile in (None, (64, 64, 32), (128, 128, 32), (256, 256, 32)):
        c = tbl.gemm(ad, bd, out_dtype=torch.float32, tile=tile)
        torch.cuda.synchronize()
        assert np.array_equal(host64(c), ref), tile
    c16 = tbl.gemm(ad, bd, tile=(256, 256, 32), persistent=True)
    torch.cuda.synchronize()
    check_gemm(host64(c16), a, b, "bf16", BIG, "bf16", what="K = 2^20, bf16 out")


def test_max_m_static_and_dynamic():
    # 2^20 rows: 4096 tiles of 256 x 256 in one grid column (64 of its 256 columns exist); K of
    # nine 32-deep steps, the fewest the dynamic schedule accepts
    M, N, K = BIG, 64, 264
    a, b = _ints(M, N, K, 73)
    ad, bd = dev16(a, "bf16"), dev16(b, "bf16")
    assert tbl.gemm_tile_shape(M, N, K)[0] == 256
    rows = np.unique(np.concatenate([np.arange(256), np.linspace(0, M - 1, 1024).astype(np.int64),
                                     np.arange(M - 300, M)]))
    ref = og.gemm_rows(a, b, "bf16", rows)
    base = tbl.gemm(ad, bd, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(host64(base)[rows], ref)
    for mode, g in ((tm.SERPENTINE | tm.XCD_REMAP, 8), (tm.PANEL, 4)):
        c = tbl.gemm(ad, bd, out_dtype=torch.float32, mode=mode, group=g, persistent=True)
        torch.cuda.synchronize()
        assert torch.equal(c, base), mode
    P = tbl.default_num_programs(M, N, K, tbl.BF16, persistent=True)
    dyn = tbl.gemm_dynamic(ad, bd, out_dtype=torch.float32, mode=tm.PANEL | tm.XCD_REMAP, group=8,
                           workspace=tbl.dynamic_workspace(P))
    torch.cuda.synchronize()
    assert torch.equal(dyn, base)


def test_max_n():
    # 2^20 columns: 4096 tiles of 256 x 256 in one grid row (64 of its 256 rows exist); every row
    # of C is checked
    M, N, K = 64, BIG, 64
    a, b = _ints(M, N, K, 75)
    ad, bd = dev16(a, "bf16"), dev16(b, "bf16")
    ref = og.gemm_rows(a, b, "bf16", np.arange(M))
    for mode, g, pers in ((tm.ROW, 1, False), (tm.PANEL | tm.XCD_REMAP, 8, True)):
        c = tbl.gemm(ad, bd, out_dtype=torch.float32, mode=mode, group=g, persistent=pers)
        torch.cuda.synchronize()
        assert np.array_equal(host64(c), ref), mode


def test_max_k_elementwise_path():
    # N and K not multiples of 8 take the general path; K one below the maximum
    M, N, K = 3, 5, BIG - 1
    a, b = _ints(M, N, K, 77)
    ad, bd = dev16(a, "bf16"), dev16(b, "bf16")
    c = tbl.gemm(ad, bd, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(host64(c), og.gemm_rows(a, b, "bf16", np.arange(M)))


@pytest.mark.parametrize("shape", [(BIG, 64), (64, BIG)])
def test_transpose_max_dims(shape):
    x = synth.i32_uniform(shape, 13)
    want = oracle_transpose(x)
    xd = torch.from_numpy(x).cuda()
    out = torch.empty((shape[1], shape[0]), dtype=torch.int32, device="cuda")
    for layout in (tbl.T_NAIVE, tbl.T_PADDED, tbl.T_XOR):
        out.fill_(0)
        tbl.transpose_i32(xd, out=out, layout=layout)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), want), layout
