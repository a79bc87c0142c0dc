"""GPU parity through the C ABI alone: tests/c_consumer/gemm_consumer.c (built by
__graft_entry__.build() with gcc against include/tbl.h, libtbl.so and the HIP runtime's C API; no
Python and no torch in that process) runs GEMMs and a transpose on the GPU, and its outputs equal
the oracle: the GEMM of "CUDA Thread Block Swizzle" (section "CUDA Thread Block Swizzle
Benchmark") on integer inputs with fp32 output, exact; the int32 transpose of "CUDA Swizzle & bank
conflict" (section "Case Study / Matrix Transpose"), bit for bit."""

import os
import subprocess

import numpy as np
import pytest

import thread_block_lds_amd as tbl
from oracle import gemm as og
from oracle import tile_maps as tm
from oracle.transpose import transpose_i32
from thread_block_lds_amd import synth

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_consumer", "_build", "gemm_consumer")


def _run(args):
    if not os.path.exists(EXE):
        raise RuntimeError(f"{EXE} is not built: run __graft_entry__.build() first")
    p = subprocess.run([EXE, *map(str, args)], capture_output=True, text=True, timeout=120)
    assert p.returncode == 0, p.stderr


@pytest.mark.parametrize("M,N,K,mode,group,pers", [
    (512, 512, 512, tm.PANEL, 4, 0), (4096, 4096, 256, tm.SERPENTINE | tm.XCD_REMAP, 8, 1),
    (300, 136, 520, tm.ROW, 1, 0), (77, 9, 130, tm.COL, 1, 1),
])
def test_c_program_gemm_matches_oracle(tmp_path, M, N, K, mode, group, pers):
    a = synth.int_valued((M, K), M + 1, -2, 2, "bf16")
    b = synth.int_valued((K, N), N + 2, -2, 2, "bf16")
    fa, fb, fc = tmp_path / "a.bin", tmp_path / "b.bin", tmp_path / "c.bin"
    a.tofile(fa)
    b.tofile(fb)
    _run(["gemm", M, N, K, tbl.BF16_F32OUT, mode, group, pers, fa, fb, fc])
    c = np.fromfile(fc, dtype=np.float32).reshape(M, N).astype(np.float64)
    assert np.array_equal(c, og.gemm(a, b, "bf16"))


def test_c_program_transpose_matches_oracle(tmp_path):
    x = synth.i32_uniform((1024, 2048), 9)
    fx, fy = tmp_path / "x.bin", tmp_path / "y.bin"
    x.tofile(fx)
    for layout in (tbl.T_NAIVE, tbl.T_PADDED, tbl.T_XOR):
        _run(["transpose", 1024, 2048, layout, fx, fy])
        assert np.array_equal(np.fromfile(fy, dtype=np.int32).reshape(2048, 1024), transpose_i32(x)), layout
