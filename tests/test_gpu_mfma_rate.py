"""tbl_mfma_rate on the GPU: the MFMA stream computes what it claims, and reports its clock.

With every operand value equal to a (in A) and b (in B), each 16x16x32 MFMA adds 32 a b to each of
a lane's 4 accumulator elements, so after ``iters`` rounds of 32 MFMAs every lane's sink value is
32 x 4 x iters x 32 a b, exact in fp32 for the small integers used here.
"""

import pytest
import torch

import thread_block_lds_amd as tbl

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("a_val,b_val,elems", [(1.0, 1.0, 1 << 16), (1.0, 2.0, 8), (-3.0, 2.0, 1000)])
def test_constant_operands_give_exact_sums(dtype, a_val, b_val, elems):
    a = torch.full((elems,), a_val, dtype=dtype, device="cuda")
    b = torch.full((elems,), b_val, dtype=dtype, device="cuda")
    iters, wg = 50, 7
    flops, out, cycles = tbl.mfma_rate(a, b, workgroups=wg, iters=iters)
    torch.cuda.synchronize()
    assert flops == 2 * 16 * 16 * 32 * 32 * iters * 4 * wg
    want = 32 * 4 * iters * 32 * a_val * b_val
    assert torch.all(out == want), (out.min().item(), out.max().item(), want)
    cyc = cycles.cpu()
    assert cyc[0] > 0 and cyc[1] > 0
    # a 16x16x32 MFMA takes at least 16 core cycles per SIMD: 32 of them per round
    assert cyc[0] >= 32 * 16 * iters


def test_random_operands_run_and_clock_is_plausible():
    g = torch.Generator().manual_seed(0)
    a = (torch.rand(1 << 20, generator=g) * 2 - 1).to(torch.float16).cuda()
    b = (torch.rand(1 << 20, generator=g) * 2 - 1).to(torch.float16).cuda()
    flops, out, cycles = tbl.mfma_rate(a, b, workgroups=256, iters=400)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    cyc, ticks = (int(x) for x in cycles.cpu())
    ghz = cyc / (ticks / 100e6) / 1e9
    assert 0.3 < ghz < 3.5, ghz
