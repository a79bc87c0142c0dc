"""Oracle: the int32 matrix transpose that the shared-memory (LDS) transposes compute.

TEST INFRASTRUCTURE (see the package docstring): not imported by the library.

Source: "CUDA Swizzle & bank conflict" (whc-imageprocess.github.io), section
"Case Study / Matrix Transpose": the naive, padded and XOR-swizzled kernels all write element
(row, col) of the M x N input to element (col, row) of the N x M output; the shared-memory layout
only changes which banks the intermediate accesses hit.
"""

import numpy as np


def transpose_i32(x):
    """out[j][i] = in[i][j] for an int32 matrix, bit for bit."""
    x = np.asarray(x)
    if x.ndim != 2:
        raise ValueError("expected a 2-D matrix")
    rows, cols = x.shape
    out = np.empty((cols, rows), dtype=x.dtype)
    out[:, :] = x.T
    return out
