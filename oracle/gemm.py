"""Oracle: the GEMM C = A @ B that every tile order computes, in fp64.

TEST INFRASTRUCTURE (see the package docstring): not imported by the library.

Source: "CUDA Thread Block Swizzle" (leimao.github.io), benchmark script of section
"CUDA Thread Block Swizzle Benchmark": the kernel multiplies a row-major M x K matrix A by a
row-major K x N matrix B, accumulating in fp32 and casting to the output type, and the page checks
it against a plain matrix product; the tile order changes only which tile is computed when, never
the value of any output element.

Definition computed here: C[i][j] = sum over k of A[i][k] * B[k][j], with every input decoded
exactly to fp64. A product of two fp16 (11-bit significand) or two bf16 (8-bit) values is exact in
fp64, so the only rounding is in the fp64 sum, far below the fp32 accumulation error of the device
path. Inputs arrive as raw 16-bit patterns (numpy uint16), exactly the bytes the device reads.
"""

import numpy as np

F16, BF16 = "f16", "bf16"


def decode_f16(bits):
    """IEEE-754 binary16 bit patterns (uint16) -> fp64, exactly (numpy's float16 type decodes)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return bits.view(np.float16).astype(np.float64)


def decode_bf16(bits):
    """bfloat16 bit patterns (uint16) -> fp64, exactly.

    A bfloat16 value is the upper 16 bits of an IEEE-754 binary32 value, so shifting the pattern
    into the high half of a 32-bit word gives the binary32 encoding of the same number.
    """
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def decode(bits, dtype):
    if dtype == F16:
        return decode_f16(bits)
    if dtype == BF16:
        return decode_bf16(bits)
    raise ValueError(f"unknown input dtype {dtype}")


def gemm(a_bits, b_bits, dtype):
    """Full product C = A @ B in fp64. a_bits: (M, K) uint16, b_bits: (K, N) uint16."""
    a = decode(a_bits, dtype)
    b = decode(b_bits, dtype)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[0]:
        raise ValueError(f"shape mismatch {a.shape} x {b.shape}")
    return a @ b


def gemm_rows(a_bits, b_bits, dtype, rows):
    """Rows ``rows`` of C = A @ B in fp64 (the same definition, for a sample of rows)."""
    a = decode(np.asarray(a_bits)[np.asarray(rows)], dtype)
    b = decode(b_bits, dtype)
    return a @ b


def gemm_entries(a_bits, b_bits, dtype, rows, cols):
    """C[rows[q], cols[q]] for each q, each as its own fp64 dot product."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    a = decode(np.asarray(a_bits)[rows], dtype)            # (Q, K)
    b = decode(np.asarray(b_bits)[:, cols], dtype)         # (K, Q)
    return np.einsum("qk,kq->q", a, b)


def abs_products_rows(a_bits, b_bits, dtype, rows):
    """Rows ``rows`` of |A| @ |B| in fp64: for each output element the sum over k of
    |A[i][k] B[k][j]|. It bounds the rounding error of every summation order of that element's
    products: a sum of K terms, each addition rounded to a unit roundoff u, errs by at most about
    K u times it, whatever the order."""
    a = np.abs(decode(np.asarray(a_bits)[np.asarray(rows)], dtype))
    b = np.abs(decode(b_bits, dtype))
    return a @ b
