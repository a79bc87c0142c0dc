"""The Python binding refuses tensors that are not in GPU memory before any address reaches the
library (a host address passed to a kernel would fault the GPU). CPU only."""

import pytest
import torch

import thread_block_lds_amd as tbl


def test_gemm_rejects_host_tensors():
    a = torch.zeros((64, 64), dtype=torch.float16)
    b = torch.zeros((64, 64), dtype=torch.float16)
    c = torch.zeros((64, 64), dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU tensor"):
        tbl.gemm(a, b, c)
    with pytest.raises(ValueError, match="GPU tensor"):
        tbl.gemm_lds_layout(a, b, tbl.LDS_LAYOUTS[0], c)
    with pytest.raises(ValueError, match="GPU tensor"):
        tbl.gemm_dynamic(a, b, c, num_programs=4, workspace=torch.zeros(256, dtype=torch.int32))


def test_other_entry_points_reject_host_tensors():
    with pytest.raises(ValueError, match="GPU tensor"):
        tbl.mfma_rate(torch.zeros(64, dtype=torch.float16), torch.zeros(64, dtype=torch.float16))
    x = torch.zeros((64, 64), dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU tensor"):
        tbl.transpose_i32(x, out=torch.zeros((64, 64), dtype=torch.int32))
    with pytest.raises(ValueError, match="GPU tensor"):
        tbl.tile_map(tbl.ROW, 4, 4, out_m=torch.zeros(16, dtype=torch.int32),
                     out_n=torch.zeros(16, dtype=torch.int32))


def test_binding_argument_shapes():
    with pytest.raises(ValueError):
        tbl.gemm(torch.zeros((8, 16), dtype=torch.float16), torch.zeros((8, 16), dtype=torch.float16))
    with pytest.raises(TypeError):
        tbl.gemm(torch.zeros((8, 8), dtype=torch.float16), torch.zeros((8, 8), dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        tbl.gemm_dynamic(torch.zeros((8, 16), dtype=torch.float16), torch.zeros((8, 16), dtype=torch.float16))
    with pytest.raises(TypeError):
        tbl.gemm_dynamic(torch.zeros((8, 8), dtype=torch.float16), torch.zeros((8, 8), dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        tbl.transpose_i32(torch.zeros((8, 8), dtype=torch.float32))
