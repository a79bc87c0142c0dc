"""GPU parity: the int32 LDS transpose is bit-exact against the oracle in all three LDS layouts,
on the case study's 1024 x 2048 matrix, the 16384 x 16384 throughput workload, and small and
rectangular shapes; sizes that are not multiples of the 64 x 64 tile are rejected."""

import numpy as np
import pytest
import torch

import thread_block_lds_amd as tbl
from oracle.transpose import transpose_i32 as oracle_transpose
from thread_block_lds_amd import synth

pytestmark = pytest.mark.gpu

LAYOUTS = [tbl.T_NAIVE, tbl.T_PADDED, tbl.T_XOR]


@pytest.mark.parametrize("shape", [(64, 64), (64, 128), (192, 320), (128, 448), (1024, 2048), (2048, 1024)])
def test_transpose_small_and_case_study(shape):
    x = synth.i32_uniform(shape, 11)
    want = oracle_transpose(x)
    xd = torch.from_numpy(x).cuda()
    for layout in LAYOUTS:
        out = tbl.transpose_i32(xd, layout=layout)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), want), (shape, layout)


def test_transpose_16384_squared():
    n = 16384
    x = synth.i32_uniform((n, n), 12)
    want = oracle_transpose(x)
    xd = torch.from_numpy(x).cuda()
    out = torch.empty((n, n), dtype=torch.int32, device="cuda")
    for layout in LAYOUTS:
        out.fill_(0)
        tbl.transpose_i32(xd, out=out, layout=layout)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), want), layout


def test_transpose_rejects_ragged():
    xd = torch.zeros((100, 64), dtype=torch.int32, device="cuda")
    with pytest.raises(tbl.TblError) as e:
        tbl.transpose_i32(xd)
    assert e.value.status == tbl.ERR_SHAPE


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, (1 << 26) + 48, (1 << 32) + 4096])
def test_copy16_bit_exact(nbytes):
    # the copy that measures the transpose's read-once, write-once HBM rate: identical bytes, with
    # and without non-temporal accesses; the last size needs a second pass of the 2^20-workgroup grid
    n = nbytes // 4
    if nbytes < (1 << 30):
        x = torch.from_numpy(synth.i32_uniform((n,), 21)).cuda()
    else:
        g = torch.Generator(device="cuda")
        g.manual_seed(21)
        x = torch.randint(-2 ** 31, 2 ** 31 - 1, (n,), dtype=torch.int32, device="cuda", generator=g)
    for nt in (False, True):
        y = torch.zeros_like(x)
        tbl.copy16(x, y, nontemporal=nt)
        torch.cuda.synchronize()
        assert torch.equal(x, y), (nbytes, nt)
    del x, y
