"""The C-ABI library on the host: it loads, exports every entry point include/tbl.h declares, and
rejects invalid arguments before any HIP call (so these run without a GPU). CPU only.

Every call here fails validation; none reaches a kernel launch, so the fake device addresses used
are never dereferenced.
"""

import ctypes
import os
import re

import pytest

import thread_block_lds_amd as tbl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tbl.h")
FAKE = ctypes.c_void_p(0x10000)        # 16-byte aligned, never dereferenced
MISALIGNED = ctypes.c_void_p(0x10008)
NULL = ctypes.c_void_p(0)
# separate fake buffers, 2^44 bytes apart (more than any accepted operand), never dereferenced
FA, FB, FC, FW = (ctypes.c_void_p(i << 44) for i in (1, 2, 3, 4))


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tbl_[a-z0-9_]+)\s*\(", src)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = tbl.lib()
    declared = _declared()
    assert len(declared) >= 9
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(tbl.exported_names()) == declared
    assert tbl.version() == 107


def test_status_strings():
    for st in (0, -1, -2, -3, -4, -5, -6, -7, 1, 12345):
        assert isinstance(tbl.status_string(st), str) and tbl.status_string(st)


def _gemm(A=FA, B=FB, C=FC, M=512, N=512, K=512, dtype=0, mode=0, group=1, persistent=0, P=0):
    return tbl.lib().tbl_gemm(A, B, C, M, N, K, dtype, mode, group, persistent, P, NULL)


def _tiled(M=512, N=512, K=512, mode=0, group=1, bm=64, bn=64, bk=32, A=FA, dtype=0):
    return tbl.lib().tbl_gemm_tiled(A, FB, FC, M, N, K, dtype, mode, group, 0, 0, bm, bn, bk, NULL, NULL)


@pytest.mark.parametrize("kw,want", [
    (dict(A=NULL), tbl.ERR_INVALID_ARG), (dict(B=NULL), tbl.ERR_INVALID_ARG), (dict(C=NULL), tbl.ERR_INVALID_ARG),
    (dict(M=-1), tbl.ERR_INVALID_ARG), (dict(N=-64), tbl.ERR_INVALID_ARG), (dict(K=-8), tbl.ERR_INVALID_ARG),
    (dict(dtype=4), tbl.ERR_DTYPE), (dict(dtype=-1), tbl.ERR_DTYPE),
    (dict(mode=6), tbl.ERR_INVALID_ARG), (dict(mode=0x200), tbl.ERR_INVALID_ARG), (dict(mode=-1), tbl.ERR_INVALID_ARG),
    (dict(mode=tbl.PANEL, group=0), tbl.ERR_INVALID_ARG), (dict(mode=tbl.SERPENTINE, group=-2), tbl.ERR_INVALID_ARG),
    (dict(persistent=2), tbl.ERR_INVALID_ARG), (dict(P=-1), tbl.ERR_INVALID_ARG),
    (dict(M=(1 << 20) + 256, N=2048), tbl.ERR_SHAPE), (dict(N=(1 << 20) + 1), tbl.ERR_SHAPE),
    (dict(K=(1 << 20) + 3), tbl.ERR_SHAPE),
    (dict(M=10240, N=6144, K=2048, mode=tbl.MORTON), tbl.ERR_NOT_BIJECTIVE),
    (dict(M=10240, N=6144, K=2048, mode=tbl.XOR | tbl.XCD_REMAP), tbl.ERR_NOT_BIJECTIVE),
    (dict(M=1024, N=512, mode=tbl.XOR), tbl.ERR_NOT_BIJECTIVE),
    (dict(M=768, N=768, mode=tbl.MORTON), tbl.ERR_NOT_BIJECTIVE),   # 12 x 12 grid
    (dict(M=8000, N=7000, mode=tbl.XOR), tbl.ERR_NOT_BIJECTIVE),    # 32 x 28 padded grid

    (dict(A=MISALIGNED), tbl.ERR_ALIGN), (dict(C=MISALIGNED), tbl.ERR_ALIGN),
])
def test_gemm_validation(kw, want):
    assert _gemm(**kw) == want


def _dyn(M=2048, N=2048, K=2048, dtype=0, mode=0, group=1, P=64, ws=FW, ws_ints=None, A=FA, B=FB, C=FC,
         trace=NULL):
    if ws_ints is None:
        ws_ints = 32 + 32 * max(P, 1)
    return tbl.lib().tbl_gemm_dynamic(A, B, C, M, N, K, dtype, mode, group, P, ws, ws_ints, trace, NULL)


def test_gemm_dynamic_workspace_size():
    ws = tbl.lib().tbl_gemm_dynamic_workspace
    assert ws(1) == 64 and ws(256) == 32 + 32 * 256 and ws(65536) == 32 + 32 * 65536
    assert ws(0) == -1 and ws(-3) == -1 and ws(65537) == -1
    assert tbl.dynamic_workspace_ints(256) == 8224
    with pytest.raises(ValueError):
        tbl.dynamic_workspace_ints(0)


@pytest.mark.parametrize("kw,want", [
    (dict(A=NULL), tbl.ERR_INVALID_ARG), (dict(M=0), tbl.ERR_INVALID_ARG), (dict(dtype=7), tbl.ERR_DTYPE),
    (dict(mode=6), tbl.ERR_INVALID_ARG), (dict(mode=tbl.PANEL, group=0), tbl.ERR_INVALID_ARG),
    (dict(P=-1), tbl.ERR_INVALID_ARG), (dict(P=65537), tbl.ERR_INVALID_ARG),
    (dict(K=256), tbl.ERR_SHAPE), (dict(K=32), tbl.ERR_SHAPE), (dict(K=2044), tbl.ERR_SHAPE),
    (dict(N=2044), tbl.ERR_SHAPE), (dict(M=2048, N=1536, mode=tbl.MORTON), tbl.ERR_NOT_BIJECTIVE),
    (dict(ws=NULL), tbl.ERR_INVALID_ARG), (dict(ws=MISALIGNED), tbl.ERR_ALIGN),
    (dict(P=64, ws_ints=32 + 32 * 64 - 1), tbl.ERR_INVALID_ARG), (dict(A=MISALIGNED), tbl.ERR_ALIGN),
])
def test_gemm_dynamic_validation(kw, want):
    assert _dyn(**kw) == want


def _dyn_noalloc(A=FA, M=2048, N=2048, K=2048, dtype=0, mode=0, group=1, P=0):
    return tbl.lib().tbl_gemm_dynamic_noalloc(A, FB, FC, M, N, K, dtype, mode, group, P, NULL, NULL)


@pytest.mark.parametrize("kw,want", [
    (dict(A=NULL), tbl.ERR_INVALID_ARG), (dict(M=0), tbl.ERR_INVALID_ARG), (dict(dtype=7), tbl.ERR_DTYPE),
    (dict(mode=tbl.SERPENTINE, group=0), tbl.ERR_INVALID_ARG), (dict(P=-1), tbl.ERR_INVALID_ARG),
    (dict(K=256), tbl.ERR_SHAPE), (dict(M=2048, N=1536, mode=tbl.XOR), tbl.ERR_NOT_BIJECTIVE),
    (dict(A=MISALIGNED), tbl.ERR_ALIGN),
    # the scratch array holds TBL_NOALLOC_MAX_PROGRAMS workgroups; beyond the dynamic schedule's own
    # limit the workspace-taking entry point's error comes first
    (dict(P=tbl.NOALLOC_MAX_PROGRAMS + 1), tbl.ERR_SCRATCH), (dict(P=65536), tbl.ERR_SCRATCH),
    (dict(P=65537), tbl.ERR_INVALID_ARG),
])
def test_gemm_dynamic_noalloc_validation(kw, want):
    assert _dyn_noalloc(**kw) == want


def test_noalloc_limit_matches_header():
    src = open(HEADER).read()
    assert re.search(r"#define TBL_NOALLOC_MAX_PROGRAMS (\d+)", src).group(1) == str(tbl.NOALLOC_MAX_PROGRAMS)
    assert "scratch" in tbl.status_string(tbl.ERR_SCRATCH)


def test_empty_gemms_need_no_launch():
    """M = 0 or N = 0: C has no element; the call succeeds with nothing enqueued (no HIP call, so
    this runs without a GPU), empty buffers may be NULL, and what does not depend on the (empty)
    tile grid is still checked. K = 0 with M, N > 0 launches the fill kernel, covered on the GPU;
    here only its argument checks."""
    g = tbl.lib().tbl_gemm
    for M, N, K in [(0, 512, 512), (512, 0, 512), (0, 0, 0), (0, 7, 0), (3, 0, 0), (0, 0, 9)]:
        a = NULL if M * K == 0 else FA
        b = NULL if K * N == 0 else FB
        for persistent in (0, 1):
            assert g(a, b, NULL, M, N, K, 0, 0, 1, persistent, 0, NULL) == tbl.OK, (M, N, K)
    # Morton on an empty grid is not a question of bijectivity
    assert g(NULL, FB, NULL, 0, 512, 512, 1, tbl.MORTON, 1, 0, 0, NULL) == tbl.OK
    assert g(NULL, FB, NULL, 0, 512, 512, 7, 0, 1, 0, 0, NULL) == tbl.ERR_DTYPE
    assert g(NULL, FB, NULL, 0, 512, 512, 0, 6, 1, 0, 0, NULL) == tbl.ERR_INVALID_ARG
    assert g(NULL, FB, NULL, 0, 512, 512, 0, tbl.PANEL, 0, 0, 0, NULL) == tbl.ERR_INVALID_ARG
    assert g(NULL, FB, NULL, 0, 512, 512, 0, 0, 1, 2, 0, NULL) == tbl.ERR_INVALID_ARG
    assert g(NULL, FB, NULL, 0, 512, (1 << 20) + 1, 0, 0, 1, 0, 0, NULL) == tbl.ERR_SHAPE
    # a buffer with elements may not be NULL: B (512 x 512) here, though M = 0 leaves C empty
    assert g(NULL, NULL, NULL, 0, 512, 512, 0, 0, 1, 0, 0, NULL) == tbl.ERR_INVALID_ARG
    # K = 0: A and B may be NULL, C may not; the grid checks apply
    assert g(NULL, NULL, NULL, 512, 512, 0, 0, 0, 1, 0, 0, NULL) == tbl.ERR_INVALID_ARG
    assert g(NULL, NULL, MISALIGNED, 512, 512, 0, 0, 0, 1, 0, 0, NULL) == tbl.ERR_ALIGN
    assert g(NULL, NULL, FC, 1024, 512, 0, 0, tbl.XOR, 1, 0, 0, NULL) == tbl.ERR_NOT_BIJECTIVE
    t = tbl.lib().tbl_gemm_tiled
    assert t(NULL, FB, NULL, 0, 300, 77, 0, 0, 1, 0, 0, 128, 128, 32, NULL, NULL) == tbl.OK
    assert t(NULL, FB, NULL, 0, 300, 77, 0, 0, 1, 0, 0, 128, 64, 32, NULL, NULL) == tbl.ERR_SHAPE
    assert tbl.gemm_tile_shape(0, 0, 0) == (64, 64, 32) and tbl.gemm_tile_shape(0, 8192, 8192) == (64, 64, 32)
    # the dynamic schedule and the LDS-layout variants keep M, N, K >= 1
    assert _dyn(M=0) == tbl.ERR_INVALID_ARG and _dyn(N=0) == tbl.ERR_INVALID_ARG
    assert _dyn_noalloc(M=0) == tbl.ERR_INVALID_ARG
    assert _layout(K=0) == tbl.ERR_INVALID_ARG and _layout16(M=0) == tbl.ERR_INVALID_ARG


def _p(addr):
    return ctypes.c_void_p(addr)


def test_overlapping_buffers_rejected():
    """A buffer a call writes shares no byte with what it reads or its other outputs. Every case is
    rejected before any HIP call; the cases that pass the check are stopped by a later one (a
    misaligned workspace, TBL_ERR_ALIGN) so that nothing is launched."""
    M = N = K = 2048
    a, b = 1 << 44, 2 << 44
    a_end = a + M * K * 2
    # C on A, inside B, or reaching into B's first bytes
    assert _gemm(C=_p(a), M=M, N=N, K=K) == tbl.ERR_INVALID_ARG
    assert _gemm(C=_p(b + 4096), M=M, N=N, K=K) == tbl.ERR_INVALID_ARG
    assert _gemm(C=_p(b - M * N * 2 + 16), M=M, N=N, K=K) == tbl.ERR_INVALID_ARG
    # C right behind A, and A = B (both only read): no overlap, the workspace check comes next
    assert _dyn(C=_p(a_end), M=M, N=N, K=K, ws=MISALIGNED) == tbl.ERR_ALIGN
    assert _dyn(B=_p(a), M=M, N=N, K=K, ws=MISALIGNED) == tbl.ERR_ALIGN
    # C just in front of A: its fp16 extent ends at A, its fp32 extent reaches into A
    c = a - M * N * 2
    assert _dyn(C=_p(c), M=M, N=N, K=K, ws=MISALIGNED, dtype=tbl.F16) == tbl.ERR_ALIGN
    assert _dyn(C=_p(c), M=M, N=N, K=K, ws=MISALIGNED, dtype=tbl.F16_F32OUT) == tbl.ERR_INVALID_ARG
    # the workspace (the ints the kernels touch) against the operands and the trace
    P = 64
    need = 4 * (32 + 32 * P)
    assert _dyn(ws=_p(3 << 44), P=P) == tbl.ERR_INVALID_ARG            # on C
    assert _dyn(ws=_p(a_end - need + 16), P=P) == tbl.ERR_INVALID_ARG  # reaches A's end
    assert _dyn(ws=_p(a - need), P=P, trace=_p(a - need - 16)) == tbl.ERR_INVALID_ARG   # trace on it
    # a trace on an operand or on C
    assert _dyn(trace=_p(b + 64), ws=MISALIGNED) == tbl.ERR_INVALID_ARG
    assert tbl.lib().tbl_gemm_tiled(FA, FB, FC, 512, 512, 512, 0, 0, 1, 0, 0, 64, 64, 32, _p((3 << 44) + 8),
                                    NULL) == tbl.ERR_INVALID_ARG
    assert tbl.lib().tbl_gemm_tiled(FA, FB, FC, 512, 512, 512, 0, 0, 1, 0, 0, 64, 64, 32, FC, NULL) == tbl.ERR_INVALID_ARG
    # transpose: out on in, or overlapping its last row
    f = tbl.lib().tbl_transpose_i32
    assert f(FA, FA, 1024, 2048, 2, NULL) == tbl.ERR_INVALID_ARG
    assert f(FA, _p(a + 1024 * 2048 * 4 - 64), 1024, 2048, 2, NULL) == tbl.ERR_INVALID_ARG
    assert f(FA, _p(a - 1024 * 2048 * 4 + 16), 1024, 2048, 1, NULL) == tbl.ERR_INVALID_ARG


def test_gemm_tiled_validation():
    assert _tiled(bm=32, bn=32) == tbl.ERR_SHAPE
    assert _tiled(bm=64, bn=128) == tbl.ERR_SHAPE
    assert _tiled(bk=64) == tbl.ERR_SHAPE
    # N and K need not be multiples of 8 here (the general path); the other checks still apply
    assert _tiled(K=513, bk=64) == tbl.ERR_SHAPE and _tiled(N=515, bm=32, bn=32) == tbl.ERR_SHAPE
    assert _tiled(mode=tbl.MORTON, M=1024, N=512, bm=128, bn=128) == tbl.ERR_NOT_BIJECTIVE
    assert _tiled(A=MISALIGNED) == tbl.ERR_ALIGN
    assert _tiled(dtype=9) == tbl.ERR_DTYPE


def test_tile_map_validation():
    f = tbl.lib().tbl_tile_map
    assert f(0, 8, 8, 1, NULL, FAKE, NULL) == tbl.ERR_INVALID_ARG
    assert f(7, 8, 8, 1, FAKE, FAKE, NULL) == tbl.ERR_INVALID_ARG
    assert f(tbl.PANEL, 8, 8, 0, FAKE, FAKE, NULL) == tbl.ERR_INVALID_ARG
    assert f(0, -1, 8, 1, FAKE, FAKE, NULL) == tbl.ERR_SHAPE
    # an empty grid has an empty table: nothing written, NULL allowed, the mode still checked
    assert f(0, 0, 8, 1, NULL, NULL, NULL) == tbl.OK and f(tbl.SERPENTINE, 8, 0, 2, NULL, NULL, NULL) == tbl.OK
    assert f(tbl.PANEL, 0, 8, 0, NULL, NULL, NULL) == tbl.ERR_INVALID_ARG and f(9, 0, 0, 1, NULL, NULL, NULL) == tbl.ERR_INVALID_ARG
    assert f(0, 8, -1, 1, FAKE, FAKE, NULL) == tbl.ERR_SHAPE
    assert f(0, 1 << 16, 1 << 16, 1, FAKE, FAKE, NULL) == tbl.ERR_SHAPE     # 2^32 tiles


def test_transpose_validation():
    f = tbl.lib().tbl_transpose_i32
    assert f(NULL, FAKE, 64, 64, 0, NULL) == tbl.ERR_INVALID_ARG
    assert f(FAKE, FAKE, -64, 64, 0, NULL) == tbl.ERR_INVALID_ARG
    assert f(NULL, NULL, 0, 64, 0, NULL) == tbl.OK and f(NULL, NULL, 128, 0, 2, NULL) == tbl.OK   # no element
    assert f(NULL, NULL, 0, 64, 3, NULL) == tbl.ERR_INVALID_ARG and f(NULL, NULL, 0, 65, 0, NULL) == tbl.ERR_SHAPE
    assert f(FAKE, FAKE, 64, 64, 3, NULL) == tbl.ERR_INVALID_ARG
    assert f(FAKE, FAKE, 100, 64, 0, NULL) == tbl.ERR_SHAPE
    assert f(FAKE, FAKE, 64, 96, 2, NULL) == tbl.ERR_SHAPE
    assert f(FAKE, MISALIGNED, 64, 64, 1, NULL) == tbl.ERR_ALIGN


def test_tile_shape_rule_and_default_programs():
    # the largest square tile whose grid has at least 128 tiles, else 64
    assert tbl.gemm_tile_shape(512, 512, 512) == (64, 64, 32)         # 4 / 16 tiles
    assert tbl.gemm_tile_shape(1024, 1024, 8192) == (64, 64, 32)      # 16 / 64 tiles
    assert tbl.gemm_tile_shape(1536, 1536, 1536) == (128, 128, 32)    # 36 / 144
    assert tbl.gemm_tile_shape(2048, 2048, 8192) == (128, 128, 32)    # 64 / 256
    assert tbl.gemm_tile_shape(2560, 2560, 64) == (128, 128, 32)      # 100 / 400
    assert tbl.gemm_tile_shape(2816, 2816, 64) == (128, 128, 32)      # 121 / 484
    assert tbl.gemm_tile_shape(3072, 3072, 3072) == (256, 256, 32)    # 144
    assert tbl.gemm_tile_shape(4096, 4096, 4096) == (256, 256, 32)
    assert tbl.gemm_tile_shape(10240, 6144, 2048) == (256, 256, 32)
    assert tbl.gemm_tile_shape(256 * 127, 256, 8) == (128, 128, 32)   # 127 tiles of 256: one short
    assert tbl.gemm_tile_shape(256 * 128, 256, 8) == (256, 256, 32)   # exactly 128
    # non-persistent default needs no device: one workgroup per tile
    assert tbl.default_num_programs(512, 512, 512, persistent=False) == 64
    assert tbl.default_num_programs(8192, 8192, 8192, persistent=False) == 1024
    assert tbl.default_num_programs(10240, 6144, 2048, persistent=False) == 960
    assert tbl.default_num_programs(520, 512, 512, persistent=False) == 72     # 9 x 8 padded grid
    assert tbl.default_num_programs(1, 8, 8, persistent=False) == 1
    assert tbl.default_num_programs(520, 516, 509, persistent=False) == 81   # any N and K
    with pytest.raises(tbl.TblError):
        tbl.default_num_programs(520, (1 << 20) + 1, 512)


def _layout(layout=(4, 4, 4, 1, 4), dtype=0, M=512, N=512, K=512, A=FA, mode=0):
    return tbl.lib().tbl_gemm_lds_layout(A, FB, FC, M, N, K, dtype, mode, 1, 0, 0, *layout, NULL)


@pytest.mark.parametrize("kw,want", [
    (dict(layout=(3, 4, 4, 1, 4)), tbl.ERR_INVALID_ARG), (dict(layout=(4, 4, 4, 1, 8)), tbl.ERR_INVALID_ARG),
    (dict(layout=(4, 4, 16, 1, 4)), tbl.ERR_INVALID_ARG), (dict(layout=(0, 0, 0, 0, 0)), tbl.ERR_INVALID_ARG),
    (dict(dtype=tbl.BF16), tbl.ERR_DTYPE), (dict(dtype=tbl.F16_F32OUT), tbl.ERR_DTYPE), (dict(dtype=7), tbl.ERR_DTYPE),
    (dict(A=NULL), tbl.ERR_INVALID_ARG), (dict(N=500), tbl.ERR_SHAPE), (dict(A=MISALIGNED), tbl.ERR_ALIGN),
    (dict(M=768, N=512, mode=tbl.XOR), tbl.ERR_NOT_BIJECTIVE),
])
def test_gemm_lds_layout_rejects(kw, want):
    assert _layout(**kw) == want



def _rate(A=FAKE, B=FAKE, elems=1 << 20, dtype=0, wg=256, iters=100, out=FAKE, cyc=FAKE):
    return tbl.lib().tbl_mfma_rate(A, B, elems, dtype, wg, iters, out, cyc, NULL)


@pytest.mark.parametrize("kw,want", [
    (dict(A=NULL), tbl.ERR_INVALID_ARG), (dict(B=NULL), tbl.ERR_INVALID_ARG),
    (dict(out=NULL), tbl.ERR_INVALID_ARG), (dict(cyc=NULL), tbl.ERR_INVALID_ARG),
    (dict(dtype=4), tbl.ERR_DTYPE), (dict(dtype=-1), tbl.ERR_DTYPE),
    (dict(elems=7), tbl.ERR_INVALID_ARG), (dict(wg=0), tbl.ERR_INVALID_ARG),
    (dict(wg=65537), tbl.ERR_INVALID_ARG), (dict(iters=0), tbl.ERR_INVALID_ARG),
    (dict(iters=(1 << 24) + 1), tbl.ERR_INVALID_ARG), (dict(A=MISALIGNED), tbl.ERR_ALIGN),
    (dict(B=MISALIGNED), tbl.ERR_ALIGN),
])
def test_mfma_rate_rejects(kw, want):
    assert _rate(**kw) == want


def _layout16(layout=(2, 4, 0, 0, 0), dtype=0, M=512, N=512, K=512, A=FA):
    return tbl.lib().tbl_gemm_lds_layout16(A, FB, FC, M, N, K, dtype, 0, 1, 0, 0, *layout, NULL)


@pytest.mark.parametrize("kw,want", [
    (dict(layout=(8, 4, 0, 0, 0)), tbl.ERR_INVALID_ARG), (dict(layout=(4, 4, 4, 1, 4)), tbl.ERR_INVALID_ARG),
    (dict(layout=(2, 4, 0, 0, 1)), tbl.ERR_INVALID_ARG), (dict(dtype=tbl.BF16), tbl.ERR_DTYPE),
    (dict(A=NULL), tbl.ERR_INVALID_ARG), (dict(N=500), tbl.ERR_SHAPE), (dict(A=MISALIGNED), tbl.ERR_ALIGN),
])
def test_gemm_lds_layout16_rejects(kw, want):
    assert _layout16(**kw) == want


def _copy(src=FAKE, dst=ctypes.c_void_p(0x20000), nbytes=4096, nt=0):
    return tbl.lib().tbl_copy16(src, dst, nbytes, nt, NULL)


@pytest.mark.parametrize("kw,want", [
    (dict(src=NULL), tbl.ERR_INVALID_ARG), (dict(dst=NULL), tbl.ERR_INVALID_ARG),
    (dict(nbytes=-16), tbl.ERR_INVALID_ARG), (dict(nbytes=0, src=NULL, dst=NULL), tbl.OK),
    (dict(nt=2), tbl.ERR_INVALID_ARG), (dict(nt=-1), tbl.ERR_INVALID_ARG),
    (dict(nbytes=4100), tbl.ERR_SHAPE), (dict(nbytes=(1 << 40) + 16), tbl.ERR_SHAPE),
    (dict(src=MISALIGNED), tbl.ERR_ALIGN), (dict(dst=ctypes.c_void_p(0x20008)), tbl.ERR_ALIGN),
    # overlapping ranges, either way round, and the same buffer
    (dict(dst=ctypes.c_void_p(0x10000 + 4080)), tbl.ERR_INVALID_ARG),
    (dict(src=ctypes.c_void_p(0x20000 + 16), dst=ctypes.c_void_p(0x20000)), tbl.ERR_INVALID_ARG),
    (dict(dst=FAKE), tbl.ERR_INVALID_ARG),
])
def test_copy16_rejects(kw, want):
    assert _copy(**kw) == want
