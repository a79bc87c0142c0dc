"""Pins of the GEMM oracle (fp16/bf16 decoding and the fp64 product). CPU only.

Pins: the IEEE-754 binary16 and bfloat16 definitions at hand-picked bit patterns; a brute-force
triple loop with exactly rounded sums (math.fsum) on tiny random shapes; exact integer products;
the identity matrix; and the sampled-row / sampled-entry helpers against the full product.
"""

import math

import numpy as np
import pytest

from oracle import gemm as og
from thread_block_lds_amd import synth


F16_CASES = [(0x3C00, 1.0), (0xBC00, -1.0), (0x4000, 2.0), (0x3555, 0.333251953125),
             (0x7BFF, 65504.0), (0x0001, 2.0 ** -24), (0x0400, 2.0 ** -14), (0x03FF, 1023 * 2.0 ** -24),
             (0x8000, -0.0), (0x3800, 0.5), (0xC500, -5.0)]
BF16_CASES = [(0x3F80, 1.0), (0xC000, -2.0), (0x4049, 3.140625), (0x3F00, 0.5),
              (0x7F7F, (2 - 2.0 ** -7) * 2.0 ** 127), (0x0080, 2.0 ** -126), (0x0001, 2.0 ** -133),
              (0xBE80, -0.25)]


def test_decode_f16_definition():
    for bits, val in F16_CASES:
        got = og.decode_f16(np.array([bits], dtype=np.uint16))[0]
        assert got == val and math.copysign(1.0, got) == math.copysign(1.0, val), hex(bits)


def test_decode_bf16_definition():
    for bits, val in BF16_CASES:
        assert og.decode_bf16(np.array([bits], dtype=np.uint16))[0] == val, hex(bits)


def _decode_by_fields(bits, exp_bits, man_bits):
    """binary format decoding from its fields: sign, biased exponent, fraction."""
    sign = -1.0 if bits >> (exp_bits + man_bits) else 1.0
    e = (bits >> man_bits) & ((1 << exp_bits) - 1)
    f = bits & ((1 << man_bits) - 1)
    bias = (1 << (exp_bits - 1)) - 1
    if e == 0:
        return sign * f * 2.0 ** (1 - bias - man_bits)
    return sign * (1 + f / 2.0 ** man_bits) * 2.0 ** (e - bias)


def test_decode_all_finite_patterns_by_fields():
    for bits in range(0, 1 << 16, 7):
        if ((bits >> 10) & 0x1F) != 0x1F:
            assert og.decode_f16(np.array([bits], np.uint16))[0] == _decode_by_fields(bits, 5, 10)
        if ((bits >> 7) & 0xFF) != 0xFF:
            assert og.decode_bf16(np.array([bits], np.uint16))[0] == _decode_by_fields(bits, 8, 7)


def _brute(a, b):
    M, K = a.shape
    N = b.shape[1]
    return np.array([[math.fsum(float(a[i, k]) * float(b[k, j]) for k in range(K)) for j in range(N)]
                     for i in range(M)])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(1, 1, 1), (2, 3, 5), (7, 1, 4), (17, 13, 11), (16, 16, 16), (5, 9, 17)])
def test_gemm_vs_brute_force(dtype, shape):
    M, N, K = shape
    if dtype == "f16":
        a = synth.f16_uniform((M, K), 3)
        b = synth.f16_uniform((K, N), 4)
    else:
        a = synth.bf16_normal((M, K), 3)
        b = synth.bf16_normal((K, N), 4)
    c = og.gemm(a, b, dtype)
    ref = _brute(og.decode(a, dtype), og.decode(b, dtype))
    assert c.shape == (M, N)
    assert np.allclose(c, ref, rtol=1e-13, atol=1e-13)


def test_gemm_integer_exact():
    M, N, K = 9, 11, 64
    a = synth.int_valued((M, K), 5, -3, 3, "f16")
    b = synth.int_valued((K, N), 6, -3, 3, "f16")
    ai = og.decode_f16(a).astype(np.int64)
    bi = og.decode_f16(b).astype(np.int64)
    want = [[sum(int(ai[i, k]) * int(bi[k, j]) for k in range(K)) for j in range(N)] for i in range(M)]
    assert np.array_equal(og.gemm(a, b, "f16"), np.array(want, dtype=np.float64))


def test_gemm_identity():
    K = 32
    eye = np.eye(K, dtype=np.float16).view(np.uint16)
    b = synth.f16_uniform((K, 24), 9)
    assert np.array_equal(og.gemm(eye, b, "f16"), og.decode_f16(b))


def test_gemm_shape_mismatch():
    with pytest.raises(ValueError):
        og.gemm(np.zeros((2, 3), np.uint16), np.zeros((4, 2), np.uint16), "f16")


def test_sampled_helpers_match_full():
    a = synth.f16_uniform((40, 33), 1)
    b = synth.f16_uniform((33, 29), 2)
    full = og.gemm(a, b, "f16")
    rows = [0, 7, 39]
    assert np.allclose(og.gemm_rows(a, b, "f16", rows), full[rows], rtol=1e-14, atol=1e-14)
    r = np.array([0, 5, 39, 12])
    c = np.array([28, 0, 3, 14])
    assert np.allclose(og.gemm_entries(a, b, "f16", r, c), full[r, c], rtol=1e-14, atol=1e-14)


def test_synth_bf16_rounding_is_nearest_even():
    # 1 + 2^-8 sits halfway between two bf16 values (1 and 1 + 2^-7): ties go to the even one, 1.
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -9)], dtype=np.float32)
    bits = synth.f32_to_bf16_bits(x)
    assert list(og.decode_bf16(bits)) == [1.0, 1.0 + 2.0 ** -6, -1.0]


def test_abs_products_by_hand_and_properties():
    # A = [[1, -2]], B = [[3], [4]] (fp16): products 3 and -8; their absolute sum is 11, the product -5
    a = np.array([[1.0, -2.0]], dtype=np.float16).view(np.uint16)
    b = np.array([[3.0], [4.0]], dtype=np.float16).view(np.uint16)
    assert og.abs_products_rows(a, b, "f16", [0])[0, 0] == 11.0
    assert og.gemm_rows(a, b, "f16", [0])[0, 0] == -5.0
    rng = np.random.default_rng(4)
    x = rng.standard_normal((40, 70)).astype(np.float16)
    y = rng.standard_normal((70, 30)).astype(np.float16)
    rows = [0, 7, 39]
    # nonnegative operands: the same as the product
    xa, ya = np.abs(x).view(np.uint16), np.abs(y).view(np.uint16)
    assert np.array_equal(og.abs_products_rows(xa, ya, "f16", rows), og.gemm_rows(xa, ya, "f16", rows))
    # the triangle inequality: never below the product's magnitude
    xs, ys = x.view(np.uint16), y.view(np.uint16)
    assert np.all(og.abs_products_rows(xs, ys, "f16", rows) >= np.abs(og.gemm_rows(xs, ys, "f16", rows)))
