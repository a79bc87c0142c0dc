"""GPU parity of tbl_gemm_lds_layout and tbl_gemm_lds_layout16: every compiled operand-layout
variant of the 256x256x32 fp16
GEMM returns the oracle's product within the fp16-output bar and exactly the bits of the default
layout (the layout moves operands around in LDS; it never changes which values are multiplied or
in which k order they are summed).

Shapes: 300 x 520 x 264 (partial tiles on both edges and a partial k step) against the full fp64
oracle; 1100 x 1032 x 2056 and 4096^3 (row-major and panel orders) against the default kernel bit
for bit.
"""

import numpy as np
import pytest
import torch

import thread_block_lds_amd as tbl
from _helpers import check_gemm, dev16, host64
from oracle import tile_maps as tm
from thread_block_lds_amd import synth

pytestmark = pytest.mark.gpu

TILE = (256, 256, 32)


def test_layout_list():
    assert len(set(tbl.LDS_LAYOUTS)) == len(tbl.LDS_LAYOUTS) == 12
    assert tbl.LDS_LAYOUTS[0] == (4, 4, 4, 1, 4)


@pytest.mark.parametrize("layout", tbl.LDS_LAYOUTS)
def test_layout_matches_oracle_on_ragged_shape(layout):
    M, N, K = 300, 520, 264
    a, b = synth.gemm_operands(M, N, K, "f16", "uniform", seed=11)
    ad, bd = dev16(a, "f16"), dev16(b, "f16")
    c = tbl.gemm_lds_layout(ad, bd, layout, mode=tm.PANEL, group=2)
    torch.cuda.synchronize()
    check_gemm(host64(c), a, b, "f16", K, "f16", what=str(layout))
    ref = tbl.gemm(ad, bd, mode=tm.PANEL, group=2, tile=TILE)
    torch.cuda.synchronize()
    assert torch.equal(c, ref), layout


@pytest.mark.parametrize("M,N,K,mode,group", [(1100, 1032, 2056, tm.SERPENTINE, 2),
                                              (4096, 4096, 4096, tm.ROW, 1),
                                              (4096, 4096, 4096, tm.PANEL | tm.XCD_REMAP, 8)])
def test_layouts_bit_identical_to_default(M, N, K, mode, group):
    a, b = synth.gemm_operands(M, N, K, "f16", "uniform", seed=12)
    ad, bd = dev16(a, "f16"), dev16(b, "f16")
    ref = tbl.gemm(ad, bd, mode=mode, group=group, tile=TILE)
    torch.cuda.synchronize()
    for layout in tbl.LDS_LAYOUTS:
        c = tbl.gemm_lds_layout(ad, bd, layout, mode=mode, group=group)
        torch.cuda.synchronize()
        assert torch.equal(c, ref), layout
    # and the result is the product: sampled rows against the oracle
    rows = np.arange(0, M, max(1, M // 7))
    check_gemm(host64(ref[torch.from_numpy(rows).cuda()]), a, b, "f16", K, "f16", rows)


# ---- the 16x16x32 form (tbl_gemm_lds_layout16) ----

def test_layout16_list():
    assert len(set(tbl.LDS_LAYOUTS16)) == len(tbl.LDS_LAYOUTS16) == 6
    assert tbl.LDS_LAYOUTS16[0] == (2, 4, 0, 0, 0)


@pytest.mark.parametrize("layout", tbl.LDS_LAYOUTS16)
def test_layout16_matches_oracle_on_ragged_shape(layout):
    M, N, K = 300, 520, 264
    a, b = synth.gemm_operands(M, N, K, "f16", "uniform", seed=13)
    ad, bd = dev16(a, "f16"), dev16(b, "f16")
    c = tbl.gemm_lds_layout(ad, bd, layout, mode=tm.SERPENTINE, group=2, mfma16=True)
    torch.cuda.synchronize()
    check_gemm(host64(c), a, b, "f16", K, "f16", what=str(layout))
    ref = tbl.gemm(ad, bd, mode=tm.SERPENTINE, group=2, tile=TILE)
    torch.cuda.synchronize()
    assert torch.equal(c, ref), layout


def test_layouts16_bit_identical_to_default_at_4096():
    M = N = K = 4096
    a, b = synth.gemm_operands(M, N, K, "f16", "uniform", seed=14)
    ad, bd = dev16(a, "f16"), dev16(b, "f16")
    ref = tbl.gemm(ad, bd, mode=tm.PANEL | tm.XCD_REMAP, group=4, tile=TILE)
    torch.cuda.synchronize()
    for layout in tbl.LDS_LAYOUTS16:
        c = tbl.gemm_lds_layout(ad, bd, layout, mode=tm.PANEL | tm.XCD_REMAP, group=4, mfma16=True)
        torch.cuda.synchronize()
        assert torch.equal(c, ref), layout


def test_layout16_rejects_unknown_variant():
    a = torch.zeros((512, 512), dtype=torch.float16, device="cuda")
    with pytest.raises(tbl.TblError) as e:
        tbl.gemm_lds_layout(a, a, (8, 4, 0, 0, 0), mfma16=True)   # A must repeat every 16 rows
    assert e.value.status == tbl.ERR_INVALID_ARG
