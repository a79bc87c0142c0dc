"""GPU parity of tbl_gemm / tbl_gemm_tiled against the fp64 oracle.

Bars (see tests/_helpers.py): fp16/bf16 output |gpu - ref| <= 1e-2 + 1e-2 |ref|; fp32 output
|gpu - ref| <= 1e-4 sqrt(K) max|ref|. Integer-valued inputs make the fp32 accumulation exact, so
those tests compare bits: fp32 output equals the exact product, and fp16 / bf16 output equals the
exact product rounded to nearest even. For one tile shape every output element is accumulated by
the same code in the same k order whatever the tile order, so outputs must be bit-identical
across orders, the XCD remap, persistence and program counts.

Workloads (inputs from thread_block_lds_amd.synth, A seed s, B seed s+1):
  512^3 fp16 uniform[-1,1], 64x64 tiles (8x8 grid), every order, full oracle;
  4096^3 fp16 uniform[-1,1], 256x256 tiles (16x16 grid), row / panel 4,8,16 / Morton / XOR;
  8192^3 bf16 N(0,1)/sqrt(K), persistent group-major 8 and serpentine 8;
  10240 x 6144 x 2048 fp16, 40x24 grid, panel 8/16 and serpentine 8/16, both launch styles;
  ragged shapes, N and K included (odd N or K run the general path), every tile shape.
Large workloads are checked on sampled rows that touch every tile row (every tile column is in
every row), plus bit-identity of the whole output across orders.
"""

import numpy as np
import pytest
import torch

import thread_block_lds_amd as tbl
from _helpers import bits16, check_bound, check_gemm, check_tol, dev16, host64
from oracle import gemm as og
from oracle import tile_maps as tm
from thread_block_lds_amd import synth

pytestmark = pytest.mark.gpu


def _sample_rows(M, BM):
    """Two rows in every tile row, at offsets that vary from tile row to tile row."""
    rows = []
    for r in range(M // BM):
        rows.append(r * BM + (r * 37) % BM)
        rows.append(r * BM + (BM - 1 - (r * 11) % BM))
    return np.array(sorted(set(rows)))


def test_c1_every_order_full_oracle():
    M = N = K = 512
    a, b = synth.gemm_operands(M, N, K, "f16", "uniform", seed=0)
    ref = og.gemm(a, b, "f16")
    absprod = og.abs_products_rows(a, b, "f16", np.arange(M))
    ad, bd = dev16(a, "f16"), dev16(b, "f16")
    outs = []
    for mode, g in [(tm.ROW, 1), (tm.COL, 1), (tm.PANEL, 4), (tm.MORTON, 1), (tm.XOR, 1),
                    (tm.SERPENTINE, 2), (tm.PANEL | tm.XCD_REMAP, 4), (tm.SERPENTINE | tm.XCD_REMAP, 2)]:
        c = tbl.gemm(ad, bd, mode=mode, group=g)
        torch.cuda.synchronize()
        check_tol(host64(c), ref, K, what=f"512^3 mode {mode} g{g}")
        check_bound(host64(c), ref, absprod, K, "f16", what=f"512^3 mode {mode} g{g}")
        outs.append(c)
    for c in outs[1:]:
        assert torch.equal(c, outs[0])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("tile", [64, 128, 256])
def test_integer_inputs_exact_fp32_out(dtype, tile):
    M, N, K = 512, 768, 1024
    a = synth.int_valued((M, K), 21, -2, 2, dtype)
    b = synth.int_valued((K, N), 22, -2, 2, dtype)
    ref = og.gemm(a, b, dtype)
    c = tbl.gemm(dev16(a, dtype), dev16(b, dtype), out_dtype=torch.float32, tile=(tile, tile, 32),
                 mode=tm.PANEL, group=2)
    torch.cuda.synchronize()
    assert np.array_equal(host64(c), ref)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_output_rounding_is_nearest_even(dtype):
    # |C| up to 8*8*512 = 32768: exact in fp32, so the only rounding is the final cast
    M, N, K = 256, 256, 512
    a = synth.int_valued((M, K), 31, -8, 8, dtype)
    b = synth.int_valued((K, N), 32, -8, 8, dtype)
    exact = og.gemm(a, b, dtype)
    if dtype == "f16":
        want = exact.astype(np.float16).view(np.uint16)
    else:
        want = synth.f32_to_bf16_bits(exact.astype(np.float32))
    for tile in (64, 256):
        c = tbl.gemm(dev16(a, dtype), dev16(b, dtype), tile=(tile, tile, 32))
        torch.cuda.synchronize()
        assert np.array_equal(bits16(c), want), tile


@pytest.mark.parametrize("dtype,dist", [("f16", "uniform"), ("bf16", "normal")])
@pytest.mark.parametrize("out_dtype", [None, torch.float32])
def test_tile_shapes_bit_identical(dtype, dist, out_dtype):
    # the 64 and 128 kernels take 16-deep 32x32x16 MFMA steps, the 256 kernel 32-deep 16x16x32
    # ones; both accumulate each element over k in ascending order in fp32, and the results agree
    # bit for bit (ragged in every dimension, K tail included)
    M, N, K = 700, 584, 1000
    a, b = synth.gemm_operands(M, N, K, dtype, dist, seed=77)
    ad, bd = dev16(a, dtype), dev16(b, dtype)
    outs = {}
    for tile in (64, 128, 256):
        outs[tile] = tbl.gemm(ad, bd, tile=(tile, tile, 32), out_dtype=out_dtype)
    torch.cuda.synchronize()
    rows = _sample_rows(M, 64)
    check_gemm(host64(outs[256])[rows], a, b, dtype, K, "f32" if out_dtype is not None else dtype, rows,
               what=f"{dtype} tile 256")
    assert torch.equal(outs[64], outs[256]) and torch.equal(outs[128], outs[256])


@pytest.mark.parametrize("tile", [64, 128, 256])
def test_schedule_variants_bit_identical(tile):
    M = N = 1024
    K = 512
    a, b = synth.gemm_operands(M, N, K, "f16", "uniform", seed=5)
    ad, bd = dev16(a, "f16"), dev16(b, "f16")
    T = (M // tile) * (N // tile)
    base = tbl.gemm(ad, bd, tile=(tile, tile, 32))
    torch.cuda.synchronize()
    rows = _sample_rows(M, tile)
    check_gemm(host64(base)[rows], a, b, "f16", K, "f16", rows, what=f"tile {tile}")
    for mode, g in [(tm.COL, 1), (tm.PANEL, 3), (tm.MORTON, 1), (tm.XOR, 1), (tm.SERPENTINE, 3)]:
        for remap in (0, tm.XCD_REMAP):
            for persistent, P in [(0, 0), (1, 0), (0, 1), (0, 7), (1, 13), (0, T + 5)]:
                c = tbl.gemm(ad, bd, tile=(tile, tile, 32), mode=mode | remap, group=g,
                             persistent=persistent, num_programs=P)
                torch.cuda.synchronize()
                assert torch.equal(c, base), (mode, remap, persistent, P)


@pytest.mark.parametrize("tile", [64, 256])
def test_cluster_orders_bit_identical(tile):
    # the two-level order only decides which workgroup computes which tile, and when
    M, N, K = 8 * tile, 4 * tile, 256
    a, b = synth.gemm_operands(M, N, K, "f16", "uniform", seed=6)
    ad, bd = dev16(a, "f16"), dev16(b, "f16")
    base = tbl.gemm(ad, bd, tile=(tile, tile, 32))
    torch.cuda.synchronize()
    rows = _sample_rows(M, tile)
    check_gemm(host64(base)[rows], a, b, "f16", K, "f16", rows, what=f"tile {tile}")
    for mode, g, (cm, cn) in [(tm.ROW, 1, (2, 1)), (tm.PANEL, 2, (2, 2)), (tm.SERPENTINE, 2, (1, 2)),
                              (tm.MORTON, 1, (2, 1)), (tm.COL, 1, (4, 4))]:
        for remap in (0, tm.XCD_REMAP):
            for persistent in (False, True):
                c = tbl.gemm(ad, bd, tile=(tile, tile, 32), mode=mode | remap | tbl.cluster(cm, cn),
                             group=g, persistent=persistent)
                torch.cuda.synchronize()
                assert torch.equal(c, base), (mode, remap, cm, cn, persistent)
    # a cluster that does not tile the grid is rejected
    with pytest.raises(tbl.TblError):
        tbl.gemm(ad, bd, tile=(tile, tile, 32), mode=tm.ROW | tbl.cluster(3, 1))


def test_c2_4096_fp16_orders():
    M = N = K = 4096
    a, b = synth.gemm_operands(M, N, K, "f16", "uniform", seed=0)
    ad, bd = dev16(a, "f16"), dev16(b, "f16")
    rows = _sample_rows(M, 256)
    ref = og.gemm_rows(a, b, "f16", rows)
    absprod = og.abs_products_rows(a, b, "f16", rows)
    base = None
    for mode, g in [(tm.ROW, 1), (tm.PANEL, 4), (tm.PANEL, 8), (tm.PANEL, 16), (tm.MORTON, 1), (tm.XOR, 1)]:
        for remap in (0, tm.XCD_REMAP):
            c = tbl.gemm(ad, bd, mode=mode | remap, group=g)
            torch.cuda.synchronize()
            if base is None:
                base = c
                check_tol(host64(c)[rows], ref, K, what="4096^3 row")
                check_bound(host64(c)[rows], ref, absprod, K, "f16", what="4096^3 row")
            else:
                assert torch.equal(c, base), (mode, g, remap)
    c32 = tbl.gemm(ad, bd, out_dtype=torch.float32, mode=tm.PANEL, group=8)
    torch.cuda.synchronize()
    check_tol(host64(c32)[rows], ref, K, f32_out=True, what="4096^3 fp32 out")
    check_bound(host64(c32)[rows], ref, absprod, K, "f32", what="4096^3 fp32 out")


def test_c3_8192_bf16_persistent():
    M = N = K = 8192
    a, b = synth.gemm_operands(M, N, K, "bf16", "normal", seed=0)
    ad, bd = dev16(a, "bf16"), dev16(b, "bf16")
    rows = _sample_rows(M, 256)
    ref = og.gemm_rows(a, b, "bf16", rows)
    absprod = og.abs_products_rows(a, b, "bf16", rows)
    base = None
    for mode in (tm.PANEL, tm.SERPENTINE, tm.PANEL | tm.XCD_REMAP, tm.SERPENTINE | tm.XCD_REMAP):
        c = tbl.gemm(ad, bd, mode=mode, group=8, persistent=True)
        torch.cuda.synchronize()
        if base is None:
            base = c
            check_tol(host64(c)[rows], ref, K, what="8192^3 bf16")
            # the outputs' spread is about 0.011, so the fixed bar above is one sigma wide; this
            # one is about 6e-4 here
            check_bound(host64(c)[rows], ref, absprod, K, "bf16", what="8192^3 bf16")
        else:
            assert torch.equal(c, base), mode


def test_c3_integer_exact_full_k_loop():
    # the 8192^3 workload's launch (persistent, CUs x occupancy programs, four tiles each, 256
    # k steps per tile) on integer inputs in [-2, 2] with fp32 output: every partial sum is an
    # integer of magnitude <= 4 K = 32768 < 2^24, so the result is exact and must equal the oracle
    # bit for bit; a skipped, doubled or misplaced k step anywhere in the loop would show
    M = N = K = 8192
    a = synth.int_valued((M, K), 61, -2, 2, "bf16")
    b = synth.int_valued((K, N), 62, -2, 2, "bf16")
    ad, bd = dev16(a, "bf16"), dev16(b, "bf16")
    rows = _sample_rows(M, 256)
    ref = og.gemm_rows(a, b, "bf16", rows)
    static = tbl.gemm(ad, bd, out_dtype=torch.float32, mode=tm.SERPENTINE | tm.XCD_REMAP, group=8,
                      persistent=True)
    torch.cuda.synchronize()
    assert np.array_equal(host64(static)[rows], ref)
    P = tbl.default_num_programs(M, N, K, tbl.BF16, persistent=True)
    for mode in (tm.PANEL | tm.XCD_REMAP, tm.PANEL):
        ws = tbl.dynamic_workspace(P)
        dyn = tbl.gemm_dynamic(ad, bd, out_dtype=torch.float32, mode=mode, group=8, workspace=ws)
        torch.cuda.synchronize()
        assert int(ws[9].item()) == 0
        assert torch.equal(dyn, static), mode


def test_c4_rectangular_partial_groups():
    M, N, K = 10240, 6144, 2048
    a, b = synth.gemm_operands(M, N, K, "f16", "uniform", seed=0)
    ad, bd = dev16(a, "f16"), dev16(b, "f16")
    rows = _sample_rows(M, 256)
    base = None
    for mode, g in [(tm.PANEL, 8), (tm.PANEL, 16), (tm.SERPENTINE, 8), (tm.SERPENTINE, 16)]:
        for persistent in (False, True):
            c = tbl.gemm(ad, bd, mode=mode, group=g, persistent=persistent)
            torch.cuda.synchronize()
            if base is None:
                base = c
                check_gemm(host64(c)[rows], a, b, "f16", K, "f16", rows, what="10240x6144x2048")
            else:
                assert torch.equal(c, base), (mode, g, persistent)
    with pytest.raises(tbl.TblError) as e:
        tbl.gemm(ad, bd, mode=tm.MORTON)
    assert e.value.status == tbl.ERR_NOT_BIJECTIVE


@pytest.mark.parametrize("mode,g,persistent,P", [(tm.PANEL, 8, True, 0), (tm.SERPENTINE, 8, True, 0),
                                                 (tm.PANEL | tm.XCD_REMAP, 8, True, 0),
                                                 (tm.ROW, 1, False, 0), (tm.XOR, 1, False, 100)])
def test_trace_matches_oracle_schedule(mode, g, persistent, P):
    M = N = 8192
    K = 32
    a, b = synth.gemm_operands(M, N, K, "f16", "uniform", seed=3)
    T = (M // 256) * (N // 256)
    trace = torch.full((8 * T,), -1, dtype=torch.int32, device="cuda")
    tbl.gemm(dev16(a, "f16"), dev16(b, "f16"), mode=mode, group=g, persistent=persistent,
             num_programs=P, trace=trace)
    torch.cuda.synchronize()
    tr = trace.cpu().numpy().reshape(T, 8).astype(np.int64)
    programs = P or (tbl.default_num_programs(M, N, K, persistent=persistent))
    om, on = tm.tile_table(mode, M // 256, N // 256, g)
    for t in range(T):
        assert tr[t, 0] == t % programs and tr[t, 1] == t // programs, t
    assert np.array_equal(tr[:, 2], om) and np.array_equal(tr[:, 3], on)
    xcc = tr[:, 4]
    assert np.all((xcc >= 0) & (xcc < 8))
    for p in range(min(programs, T)):
        assert len(set(xcc[p::programs])) == 1, p           # a workgroup never changes XCD
    # the XCD remap rests on round-robin dispatch: workgroup p runs on XCD p mod 8
    rr = np.mean(xcc[:min(programs, T)] == np.arange(min(programs, T)) % 8)
    assert rr == 1.0, f"only {rr:.3f} of the workgroups ran on XCD (program mod 8)"
    # timing fields: a program's tiles start in iteration order, each after the previous k loop
    ticks = tr[:, 6] & 0xFFFFFFFF
    start = tr[:, 7] & 0xFFFFFFFF
    assert np.all(ticks > 0)
    for t in range(T - programs):
        gap = (start[t + programs] - start[t]) % (1 << 32)
        assert ticks[t] <= gap < (1 << 31), t


RAGGED = [  # (M, N, K, tile): partial tiles at every edge, K tails of 8 .. 24, tiny and single-tile
    (1, 8, 8, 64), (3, 8, 40, 64), (100, 136, 104, 64), (65, 72, 8, 64), (257, 264, 1000, 64),
    (300, 200, 72, 128), (1000, 1000, 1000, 128), (129, 392, 520, 128),
    (513, 264, 136, 256), (1100, 1032, 2056, 256), (255, 520, 4104, 256),
]


@pytest.mark.parametrize("M,N,K,tile", RAGGED)
def test_ragged_edges_full_oracle(M, N, K, tile):
    a, b = synth.gemm_operands(M, N, K, "f16", "uniform", seed=M + N + K)
    ad, bd = dev16(a, "f16"), dev16(b, "f16")
    c = tbl.gemm(ad, bd, tile=(tile, tile, 32), mode=tm.PANEL, group=2)
    torch.cuda.synchronize()
    check_gemm(host64(c), a, b, "f16", K, "f16", what=f"ragged {M}x{N}x{K} tile {tile}")
    c32 = tbl.gemm(ad, bd, tile=(tile, tile, 32), out_dtype=torch.float32, mode=tm.SERPENTINE,
                   group=3, persistent=True)
    torch.cuda.synchronize()
    check_gemm(host64(c32), a, b, "f16", K, "f32", what=f"ragged fp32 {M}x{N}x{K} tile {tile}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_ragged_integer_exact_and_untouched_padding(dtype):
    # integer inputs: exact; the output is written into a larger buffer view to check that no
    # element outside C is written
    M, N, K = 300, 264, 200
    a = synth.int_valued((M, K), 41, -3, 3, dtype)
    b = synth.int_valued((K, N), 42, -3, 3, dtype)
    ref = og.gemm(a, b, dtype)
    big = torch.full((M + 64, N), 12345.0, dtype=torch.float32, device="cuda")
    c = big[:M]
    for tile in (64, 128, 256):
        big.fill_(12345.0)
        tbl.gemm(dev16(a, dtype), dev16(b, dtype), c=c, out_dtype=torch.float32, tile=(tile, tile, 32))
        torch.cuda.synchronize()
        assert np.array_equal(host64(c), ref), tile
        assert torch.all(big[M:] == 12345.0), tile


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("tile", [64, 128, 256])
def test_ragged_integer_16bit_out_is_the_rounded_exact_sum(dtype, tile):
    # integer inputs: the fp32 sums are exact, so the 16-bit output must be the exact sum rounded
    # to nearest even in the output type (torch's CPU conversion serves as that rounding); no
    # element outside C may be written
    M, N, K = 300, 264, 1000   # sums reach past 256 (bf16) and 2048 (fp16): rounding is exercised
    a = synth.int_valued((M, K), 43, -7, 7, dtype)
    b = synth.int_valued((K, N), 44, -7, 7, dtype)
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    want = torch.from_numpy(og.gemm(a, b, dtype)).to(tdt)
    big = torch.full((M + 64, N), -5.0, dtype=tdt, device="cuda")
    c = big[:M]
    tbl.gemm(dev16(a, dtype), dev16(b, dtype), c=c, tile=(tile, tile, 32), mode=tm.PANEL, group=2)
    torch.cuda.synchronize()
    assert torch.equal(c.cpu().view(torch.int16), want.view(torch.int16)), (dtype, tile)
    assert torch.all(big[M:] == -5.0), (dtype, tile)


# N or K not a multiple of 8: rows of A or B are not whole 16-byte chunks and the general path
# runs (every load and store masked at the edges, as the swizzle page's kernel masks them)
ODD = [(257, 263, 259), (1, 1, 1), (1000, 1001, 1003), (3, 5, 7), (64, 63, 65), (129, 130, 31),
       (300, 256, 100), (520, 8, 13), (200, 520, 97), (77, 16, 33)]


@pytest.mark.parametrize("tile", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K", ODD)
def test_odd_n_k_full_oracle(M, N, K, dtype, tile):
    a, b = synth.gemm_operands(M, N, K, dtype, "uniform" if dtype == "f16" else "normal", seed=M + 2 * N + 3 * K)
    ad, bd = dev16(a, dtype), dev16(b, dtype)
    c = tbl.gemm(ad, bd, tile=(tile, tile, 32), mode=tm.PANEL, group=2)
    c32 = tbl.gemm(ad, bd, tile=(tile, tile, 32), out_dtype=torch.float32, mode=tm.SERPENTINE, group=3,
                   persistent=True)
    torch.cuda.synchronize()
    check_gemm(host64(c), a, b, dtype, K, dtype, what=f"odd {M}x{N}x{K} {dtype} tile {tile}")
    check_gemm(host64(c32), a, b, dtype, K, "f32", what=f"odd fp32 {M}x{N}x{K} {dtype} tile {tile}")


@pytest.mark.parametrize("N", [263, 264])
@pytest.mark.parametrize("tile", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_odd_n_k_integer_exact_untouched_padding_and_schedules(dtype, tile, N):
    # integer inputs in [-7, 7]: fp32 sums are exact, 16-bit outputs the exact sum rounded to nearest
    # even; the output sits inside a larger buffer whose other elements must stay untouched; every
    # order, remap and launch style gives the same bits. N = 263 moves B element by element, N = 264
    # (a multiple of 8, K odd) in 16-byte chunks, A in both in unaligned 16-byte chunks and a last
    # partial k step
    M, K = 301, 1001
    a = synth.int_valued((M, K), 45, -7, 7, dtype)
    b = synth.int_valued((K, N), 46, -7, 7, dtype)
    exact = og.gemm(a, b, dtype)
    ad, bd = dev16(a, dtype), dev16(b, dtype)
    big = torch.full((M + 3, N), 777.0, dtype=torch.float32, device="cuda")
    c = big[:M]
    tbl.gemm(ad, bd, c=c, out_dtype=torch.float32, tile=(tile, tile, 32))
    torch.cuda.synchronize()
    assert np.array_equal(host64(c), exact)
    assert torch.all(big[M:] == 777.0)
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    want = torch.from_numpy(exact).to(tdt)
    big16 = torch.full((M + 3, N), -5.0, dtype=tdt, device="cuda")
    base = big16[:M]
    tbl.gemm(ad, bd, c=base, tile=(tile, tile, 32))
    torch.cuda.synchronize()
    assert torch.equal(base.cpu().view(torch.int16), want.view(torch.int16))
    assert torch.all(big16[M:] == -5.0)
    T = (-(-M // tile)) * (-(-N // tile))
    for mode, g in [(tm.COL, 1), (tm.PANEL, 3), (tm.SERPENTINE, 2)]:
        for remap in (0, tm.XCD_REMAP):
            for persistent, P in [(0, 0), (1, 0), (0, 1), (0, T + 3)]:
                o = tbl.gemm(ad, bd, tile=(tile, tile, 32), mode=mode | remap, group=g,
                             persistent=bool(persistent), num_programs=P)
                torch.cuda.synchronize()
                assert torch.equal(o, base), (mode, remap, persistent, P)


def test_odd_n_k_tile_shapes_bit_identical():
    # the general path takes 32-deep 16x16x32 steps in every tile shape
    M, N, K = 257, 263, 259
    a, b = synth.gemm_operands(M, N, K, "bf16", "normal", seed=8)
    ad, bd = dev16(a, "bf16"), dev16(b, "bf16")
    outs = [tbl.gemm(ad, bd, tile=(t, t, 32), out_dtype=torch.float32) for t in (64, 128, 256)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


def test_odd_n_k_trace_matches_oracle_schedule():
    M, N, K = 2000, 1999, 37
    a, b = synth.gemm_operands(M, N, K, "f16", "uniform", seed=9)
    bm, bn, _ = tbl.gemm_tile_shape(M, N, K)    # the default tile (128 x 128 here: 256 tiles)
    gm, gn = -(-M // bm), -(-N // bn)
    T = gm * gn
    trace = torch.full((8 * T,), -1, dtype=torch.int32, device="cuda")
    tbl.gemm(dev16(a, "f16"), dev16(b, "f16"), mode=tm.SERPENTINE | tm.XCD_REMAP, group=2, persistent=True,
             num_programs=24, trace=trace)
    torch.cuda.synchronize()
    tr = trace.cpu().numpy().reshape(T, 8).astype(np.int64)
    om, on = tm.tile_table(tm.SERPENTINE | tm.XCD_REMAP, gm, gn, 2)
    for t in range(T):
        assert tr[t, 0] == t % 24 and tr[t, 1] == t // 24, t
    assert np.array_equal(tr[:, 2], om) and np.array_equal(tr[:, 3], on)


def test_k_tail_does_not_mix_rows():
    # A K tail reads past the end of each row of A; those elements belong to the next row. An Inf
    # placed at the start of row 1 must only reach row 1 of C.
    # (K = 41: the general path, whose masked last k step must do the same)
    for K in (40, 41):
        M, N = 64, 64
        a = synth.f16_uniform((M, K), 51)
        b = synth.f16_uniform((K, N), 52)
        a[1, 0] = np.float16(np.inf).view(np.uint16)
        for tile in (64, 128, 256):
            c = tbl.gemm(dev16(a, "f16"), dev16(b, "f16"), out_dtype=torch.float32, tile=(tile, tile, 32))
            torch.cuda.synchronize()
            got = host64(c)
            assert np.all(np.isfinite(np.delete(got, 1, axis=0))), (K, tile)
            assert not np.all(np.isfinite(got[1])), (K, tile)


@pytest.mark.parametrize("K", [8, 24, 32, 96, 160])
@pytest.mark.parametrize("tile", [64, 256])
def test_short_k_streams_across_tiles(K, tile):
    # one to five k steps per tile: the load stream runs up to four tiles ahead of the compute, so
    # a program's later tiles load while earlier ones are still computed; every schedule must give
    # the same bits and the oracle's product
    M, N = 3 * tile - 5, 3 * tile
    a, b = synth.gemm_operands(M, N, K, "f16", "uniform", seed=K + tile)
    ad, bd = dev16(a, "f16"), dev16(b, "f16")
    base = tbl.gemm(ad, bd, tile=(tile, tile, 32), out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_gemm(host64(base), a, b, "f16", K, "f32", what=f"K {K} tile {tile}")
    for persistent, P in [(0, 1), (0, 2), (1, 4), (0, 9)]:
        c = tbl.gemm(ad, bd, tile=(tile, tile, 32), out_dtype=torch.float32, mode=tm.SERPENTINE,
                     group=2, persistent=bool(persistent), num_programs=P)
        torch.cuda.synchronize()
        assert torch.equal(c, base), (K, tile, persistent, P)


def test_binding_checks_trace_and_device():
    a = torch.zeros((512, 512), dtype=torch.float16, device="cuda")
    b = torch.zeros((512, 512), dtype=torch.float16, device="cuda")
    # 512 x 512 with 256 tiles: 4 tiles need 32 trace ints
    with pytest.raises(ValueError, match="at least 32"):
        tbl.gemm(a, b, tile=(256, 256, 32), trace=torch.zeros(31, dtype=torch.int32, device="cuda"))
    with pytest.raises(TypeError):
        tbl.gemm(a, b, tile=(256, 256, 32), trace=torch.zeros(32, dtype=torch.int64, device="cuda"))
    with pytest.raises(ValueError, match="GPU tensor"):
        tbl.gemm(a, b, c=torch.zeros((512, 512), dtype=torch.float16))
    with pytest.raises(ValueError, match="at least 16"):
        tbl.tile_map(tbl.ROW, 4, 4, out_m=torch.zeros(15, dtype=torch.int32, device="cuda"))
