"""GPU test: the C-ABI called from several host threads at once. Its only global state is the
per-device property cache, guarded by a lock, so calls from four threads, each on its own stream,
must give the same bits as the same calls made one after the other (GEMMs of every tile shape,
the general path, the dynamic schedule, tile maps and transposes; ctypes releases the
interpreter lock during each call, so the threads do overlap inside the library)."""

import threading

import numpy as np
import pytest
import torch

import thread_block_lds_amd as tbl
from oracle import tile_maps as tm
from thread_block_lds_amd import synth

from _helpers import dev16

pytestmark = pytest.mark.gpu

# (M, N, K, mode, group, persistent) per job; shapes pick the 64, 128 and 256 tiles and the
# general path (N = 100)
JOBS = [(512, 512, 512, tm.PANEL, 4, False), (2048, 2048, 512, tm.SERPENTINE | tm.XCD_REMAP, 2, True),
        (4096, 4096, 512, tm.MORTON, 1, False), (700, 100, 300, tm.ROW, 1, True),
        (2048, 2048, 1024, tm.XOR | tm.XCD_REMAP, 1, False)]


def _work(inputs, x, stream):
    """Every job on one stream; returns the outputs (on the device)."""
    out = []
    with torch.cuda.stream(stream):
        for (M, N, K, mode, g, pers), (a, b) in zip(JOBS, inputs):
            out.append(tbl.gemm(a, b, mode=mode, group=g, persistent=pers, stream=stream.cuda_stream))
        a, b = inputs[1]
        P = tbl.default_num_programs(2048, 2048, 512, tbl.F16, persistent=True)
        out.append(tbl.gemm_dynamic(a, b, mode=tm.PANEL | tm.XCD_REMAP, group=8,
                                    workspace=tbl.dynamic_workspace(P), stream=stream.cuda_stream))
        m, n, _ = tbl.tile_map(tm.SERPENTINE, 40, 24, 3, stream=stream.cuda_stream)
        out += [m, n]
        out.append(tbl.transpose_i32(x, layout=tbl.T_PADDED, stream=stream.cuda_stream))
    stream.synchronize()
    return out


def test_concurrent_host_threads_match_serial_calls():
    inputs = []
    for M, N, K, _, _, _ in JOBS:
        a, b = synth.gemm_operands(M, N, K, "f16", "uniform", seed=M + N + K)
        inputs.append((dev16(a, "f16"), dev16(b, "f16")))
    x = torch.from_numpy(synth.i32_uniform((1024, 2048), 3)).cuda()
    torch.cuda.synchronize()
    serial = _work(inputs, x, torch.cuda.Stream())
    results = [None] * 4
    errors = []

    def run(i):
        try:
            results[i] = _work(inputs, x, torch.cuda.Stream())
        except Exception as e:  # reported below, with the thread's index
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=run, args=(i,)) for i in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    for i, res in enumerate(results):
        assert len(res) == len(serial)
        for j, (got, want) in enumerate(zip(res, serial)):
            assert torch.equal(got, want), (i, j)
    # and the serial results are right where the oracle is cheap to ask: the tile map and transpose
    om, on = tm.tile_table(tm.SERPENTINE, 40, 24, 3)
    assert np.array_equal(serial[-3].cpu().numpy(), om) and np.array_equal(serial[-2].cpu().numpy(), on)
    assert np.array_equal(serial[-1].cpu().numpy(), x.cpu().numpy().T)
