"""The allocation-free entry point tbl_gemm_dynamic_noalloc (the dynamic schedule with its claim
counters and mailboxes in the library's own device array) against tbl_gemm_dynamic, the entry point
that takes a caller-owned workspace.

Two calls in a row on one GPU, the second on a smaller problem with fewer workgroups, so the second
runs on the array the first left behind: each output must be bit-identical to tbl_gemm_dynamic's
(the same kernel arithmetic), within the parity bars of the fp64 oracle (tests/_helpers.py), and
the second call's trace must show every order position run exactly once under the claim rules.
Inputs come from thread_block_lds_amd.synth (A seed s, B seed s + 1).
"""

import numpy as np
import pytest
import torch

import thread_block_lds_amd as tbl
from _helpers import check_gemm, dev16, host64
from oracle import schedule as sc
from thread_block_lds_amd import synth

pytestmark = pytest.mark.gpu

# (M, N, K, in dtype, out dtype, mode, group, num_programs, seed); the second is the smaller one
CALLS = [
    (2048, 2048, 1024, "f16", torch.float16, tbl.SERPENTINE | tbl.XCD_REMAP, 2, 0, 0),
    (768, 1280, 512, "bf16", torch.float32, tbl.PANEL, 2, 5, 4),
]


def _bits(t):
    return t.view(torch.int32 if t.dtype == torch.float32 else torch.int16)


def test_noalloc_matches_dynamic_on_two_calls():
    for M, N, K, dt, out_dtype, mode, g, P, seed in CALLS:
        a, b = synth.gemm_operands(M, N, K, dt, "uniform" if dt == "f16" else "normal", seed=seed)
        ad, bd = dev16(a, dt), dev16(b, dt)
        T = (-(-M // 256)) * (-(-N // 256))
        Pr = P or tbl.default_num_programs(M, N, K, tbl.F16, persistent=True)
        ws = tbl.dynamic_workspace(Pr)
        ref = tbl.gemm_dynamic(ad, bd, mode=mode, group=g, num_programs=P, workspace=ws,
                               out_dtype=out_dtype)
        tr = torch.full((8 * T,), -1, dtype=torch.int32, device="cuda")
        out = tbl.gemm_dynamic_noalloc(ad, bd, mode=mode, group=g, num_programs=P, out_dtype=out_dtype,
                                       trace=tr)
        torch.cuda.synchronize()
        print(f"noalloc {M}x{N}x{K} {dt} mode {mode:#x} P {Pr}", flush=True)
        assert torch.equal(_bits(out), _bits(ref)), "differs from tbl_gemm_dynamic"
        check_gemm(host64(out), a, b, dt, K, "f32" if out_dtype == torch.float32 else dt,
                   what=f"noalloc {M}x{N}x{K}")
        r = tr.cpu().numpy().reshape(T, 8).astype(np.int64)
        sc.check_dynamic_trace(r[:, 0], r[:, 1], r[:, 4], T, bool(mode & tbl.XCD_REMAP))
        assert int(ws[9].item()) == 0


def test_noalloc_rejects_beyond_its_scratch():
    a = torch.zeros((512, 512), dtype=torch.float16, device="cuda")
    with pytest.raises(tbl.TblError) as e:
        tbl.gemm_dynamic_noalloc(a, a, num_programs=tbl.NOALLOC_MAX_PROGRAMS + 1)
    assert e.value.status == tbl.ERR_SCRATCH
