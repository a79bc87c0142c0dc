"""GPU parity on IEEE special values, through every GEMM path (64, 128 and 256 tiles, the
general path for N and K that are not multiples of 8, with B element by element or in 16-byte
chunks, and the dynamic schedule): subnormal fp16 and bf16 operands, NaN and infinities among
the operands, and results beyond the fp16 range.

The oracle is the fp64 definition of C = A B that "CUDA Thread Block Swizzle" (section "CUDA
Thread Block Swizzle Benchmark") computes with fp32 accumulation, in IEEE arithmetic. Every case
is built so that fp32 holds each partial sum exactly (integer multiples of one power of two, few
enough terms), so the GPU result must equal the oracle bit for bit: a subnormal operand flushed to
zero, a NaN lost, an infinity of the wrong sign or an overflow rounded the wrong way would show.
"""

import numpy as np
import pytest
import torch

import thread_block_lds_amd as tbl
from oracle import gemm as og
from oracle import tile_maps as tm

from _helpers import host64

pytestmark = pytest.mark.gpu

# (tile, M, N, K): the three fast kernels with partial tiles, and the general path (B element by
# element for N = 9, in 16-byte chunks for N = 136 and 264 with K odd)
PATHS = [((64, 64, 32), 70, 72, 96), ((128, 128, 32), 130, 136, 64), ((256, 256, 32), 260, 264, 40),
         ((64, 64, 32), 37, 9, 77), ((128, 128, 32), 130, 136, 77), ((256, 256, 32), 260, 264, 45)]
DT = {"f16": torch.float16, "bf16": torch.bfloat16}


def _dev(x, dtype):
    """float64 numpy values (exactly representable in the 16-bit type) -> (device tensor, bits)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DT[dtype])
    assert np.array_equal(t.double().numpy(), x, equal_nan=True), "value not representable"
    return t.cuda(), t.view(torch.int16).numpy().view(np.uint16)


def _gemm(ad, bd, tile, out=torch.float32):
    c = tbl.gemm(ad, bd, out_dtype=out, tile=tile, mode=tm.PANEL | tm.XCD_REMAP, group=2)
    torch.cuda.synchronize()
    return c


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("tile,M,N,K", PATHS)
def test_subnormal_operands_exact(dtype, tile, M, N, K):
    rng = np.random.default_rng(M + N + K)
    # A: subnormal values only (integer multiples of the type's smallest subnormal, below its
    # smallest normal); B: small integers, or for bf16 small integers times 2^100 so that some
    # products are normal fp32 values and some stay subnormal
    if dtype == "f16":
        unit, span = 2.0 ** -24, 1023
    else:
        unit, span = 2.0 ** -133, 127
    a = rng.integers(-span, span + 1, size=(M, K)).astype(np.float64) * unit
    b = rng.integers(-4, 5, size=(K, N)).astype(np.float64)
    if dtype == "bf16":
        b[:, : N // 2] *= 2.0 ** 100
    ad, a_bits = _dev(a, dtype)
    bd, b_bits = _dev(b, dtype)
    ref = og.gemm_rows(a_bits, b_bits, dtype, np.arange(M))
    assert np.count_nonzero(ref) > M * N // 2
    c = host64(_gemm(ad, bd, tile))
    assert np.array_equal(c, ref), (dtype, tile, M, N, K)
    # the subnormal operand on the B side
    b2 = rng.integers(-span, span + 1, size=(K, N)).astype(np.float64) * unit
    a2 = rng.integers(-4, 5, size=(M, K)).astype(np.float64)
    ad2, a2_bits = _dev(a2, dtype)
    bd2, b2_bits = _dev(b2, dtype)
    ref2 = og.gemm_rows(a2_bits, b2_bits, dtype, np.arange(M))
    assert np.array_equal(host64(_gemm(ad2, bd2, tile)), ref2), (dtype, tile, "B subnormal")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("tile,M,N,K", PATHS)
def test_nan_and_infinity_propagate(dtype, tile, M, N, K):
    rng = np.random.default_rng(7 * M + K)
    a = rng.integers(-3, 4, size=(M, K)).astype(np.float64)
    b = rng.integers(-3, 4, size=(K, N)).astype(np.float64)
    a[1, 2] = np.nan                     # row 1 of C: NaN everywhere
    a[3, 4] = np.inf                     # row 3: +-inf by the sign of B[4, j], NaN where B[4, j] = 0
    b[4, : N // 3] = 0.0
    b[5, N - 1] = -np.inf                # column N-1: -+inf by the sign of A[i, 5], NaN where it is 0
    a[M - 1, 5] = 0.0
    a[M - 2, 6], b[6, 0] = np.inf, np.inf    # C[M-2, 0] = +inf + (row M-2 . column 0) = +inf
    ad, a_bits = _dev(a, dtype)
    bd, b_bits = _dev(b, dtype)
    with np.errstate(invalid="ignore"):   # inf * 0 and inf - inf are meant
        ref = og.gemm_rows(a_bits, b_bits, dtype, np.arange(M))
        # the oracle's matrix product keeps IEEE semantics for these values: the same masks as the
        # sum of the elementwise products, formed without a library product
        brute = (og.decode(a_bits, dtype)[:, :, None] * og.decode(b_bits, dtype)[None, :, :]).sum(axis=1)
    for f in (np.isnan, np.isposinf, np.isneginf):
        assert np.array_equal(f(ref), f(brute))
    c = host64(_gemm(ad, bd, tile))
    assert np.array_equal(np.isnan(c), np.isnan(ref))
    assert np.array_equal(np.isposinf(c), np.isposinf(ref))
    assert np.array_equal(np.isneginf(c), np.isneginf(ref))
    fin = np.isfinite(ref)
    assert np.array_equal(c[fin], ref[fin])
    assert np.isnan(ref[1]).all() and np.isnan(ref[M - 1, N - 1]) and ref[M - 2, 0] == np.inf


@pytest.mark.parametrize("tile,M,N,K", PATHS)
def test_fp16_output_overflow_rounds_to_nearest_even(tile, M, N, K):
    # C[i, j] = 2047 * 32 + r (i, j) exactly in fp32: 65504 (the largest fp16), 65519 (rounds down to
    # it), 65520 (the halfway point: ties to even, which is infinity), larger values and their
    # negatives; each must equal the oracle's exact value rounded to fp16
    rng = np.random.default_rng(M)
    a = np.zeros((M, K))
    b = np.zeros((K, N))
    a[:, 0] = 2047.0 * rng.choice([-1.0, 1.0], size=M)
    b[0, :] = 32.0
    a[:, 1] = np.resize([0.0, 15.0, 16.0, 17.0, 31.0, 32.0, 1000.0, -15.0, -16.0], M)
    b[1, :] = np.resize([1.0, 1.0, -1.0, 2.0], N)
    a[:, 2] = rng.integers(-2, 3, size=M)
    b[2, :] = rng.integers(-2, 3, size=N)
    ad, a_bits = _dev(a, "f16")
    bd, b_bits = _dev(b, "f16")
    ref = og.gemm_rows(a_bits, b_bits, "f16", np.arange(M))
    with np.errstate(over="ignore"):
        want = ref.astype(np.float16)    # round to nearest even, overflow to infinity
    assert np.isinf(want).any() and (np.abs(want) == 65504.0).any()
    c = _gemm(ad, bd, tile, out=torch.float16).cpu().numpy()
    assert np.array_equal(c.view(np.uint16), want.view(np.uint16))


def test_dynamic_schedule_special_values():
    # the dynamic schedule's kernel (K >= 257) on subnormal bf16 operands and a planted NaN
    M, N, K = 300, 264, 264
    rng = np.random.default_rng(5)
    a = rng.integers(-127, 128, size=(M, K)).astype(np.float64) * 2.0 ** -133
    b = rng.integers(-4, 5, size=(K, N)).astype(np.float64) * 2.0 ** 100
    a[7, 100] = np.nan
    ad, a_bits = _dev(a, "bf16")
    bd, b_bits = _dev(b, "bf16")
    with np.errstate(invalid="ignore"):
        ref = og.gemm_rows(a_bits, b_bits, "bf16", np.arange(M))
    P = tbl.default_num_programs(M, N, K, tbl.BF16, persistent=True)
    c = tbl.gemm_dynamic(ad, bd, out_dtype=torch.float32, mode=tm.SERPENTINE | tm.XCD_REMAP, group=2,
                         workspace=tbl.dynamic_workspace(P))
    torch.cuda.synchronize()
    c = host64(c)
    assert np.array_equal(np.isnan(c), np.isnan(ref)) and np.isnan(ref[7]).all()
    fin = ~np.isnan(ref)
    assert np.array_equal(c[fin], ref[fin])
