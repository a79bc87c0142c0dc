"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and packs them into the bit layouts the library reads
(row-major fp16 / bf16 / int32). It holds none of the GEMM, tile-order or transpose arithmetic.

Recipe (per workload):
  * fp16 GEMM operands: uniform on [-1, 1] drawn in fp32, rounded to fp16 (round to nearest even).
  * bf16 GEMM operands: standard normal drawn in fp32, scaled by ``scale`` (1/sqrt(K) for the
    8192^3 workload), rounded to bf16 (round to nearest even on the fp32 bit pattern).
  * fp16 standard-normal operands, unscaled (the 8192^3, 128 x 128 x 32 sweep of the swizzle
    page, which draws its inputs from a standard normal): N(0, 1) in fp32, rounded to fp16.
  * int32 transpose input: uniform over the full int32 range.
  * small-integer operands (exactness tests): uniform integers in [lo, hi], exactly representable.
A matrix's seed is given by the caller; the workloads use seed s for A and s + 1 for B.
"""

import numpy as np


def _rng(seed):
    return np.random.default_rng(np.random.PCG64(int(seed)))


def f32_to_bf16_bits(x):
    """Round fp32 values to bfloat16 (nearest, ties to even); returns the uint16 patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return u.astype(np.uint16)


def f16_uniform(shape, seed, lo=-1.0, hi=1.0):
    """fp16 bit patterns (uint16) of uniform[lo, hi] values."""
    x = _rng(seed).random(shape, dtype=np.float32) * np.float32(hi - lo) + np.float32(lo)
    return x.astype(np.float16).view(np.uint16)


def bf16_normal(shape, seed, scale=1.0):
    """bf16 bit patterns (uint16) of N(0, 1) * scale values."""
    x = _rng(seed).standard_normal(shape, dtype=np.float32) * np.float32(scale)
    return f32_to_bf16_bits(x)


def int_valued(shape, seed, lo, hi, dtype):
    """Bit patterns (uint16) of integers uniform in [lo, hi], in fp16 ("f16") or bf16 ("bf16")."""
    x = _rng(seed).integers(lo, hi + 1, size=shape).astype(np.float32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def i32_uniform(shape, seed):
    """int32 values uniform over the whole int32 range."""
    return _rng(seed).integers(-2**31, 2**31, size=shape, dtype=np.int64).astype(np.int32)


def gemm_operands(M, N, K, dtype, dist, seed=0):
    """(A bits (M, K), B bits (K, N)) for a GEMM workload; A uses ``seed``, B uses ``seed + 1``.

    dist "uniform": fp16 uniform[-1, 1]; dist "normal": bf16 N(0,1)/sqrt(K) (or fp16 if asked);
    dist "randn": fp16 N(0, 1), unscaled."""
    if dist == "uniform":
        if dtype != "f16":
            raise ValueError("uniform[-1,1] inputs are generated in fp16")
        return f16_uniform((M, K), seed), f16_uniform((K, N), seed + 1)
    if dist == "normal":
        s = 1.0 / np.sqrt(K)
        if dtype == "bf16":
            return bf16_normal((M, K), seed, s), bf16_normal((K, N), seed + 1, s)
        x = _rng(seed).standard_normal((M, K), dtype=np.float32) * np.float32(s)
        y = _rng(seed + 1).standard_normal((K, N), dtype=np.float32) * np.float32(s)
        return x.astype(np.float16).view(np.uint16), y.astype(np.float16).view(np.uint16)
    if dist == "randn":
        if dtype != "f16":
            raise ValueError("unscaled normal inputs are generated in fp16")
        x = _rng(seed).standard_normal((M, K), dtype=np.float32)
        y = _rng(seed + 1).standard_normal((K, N), dtype=np.float32)
        return x.astype(np.float16).view(np.uint16), y.astype(np.float16).view(np.uint16)
    raise ValueError(dist)
