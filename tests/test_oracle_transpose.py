"""Pins of the transpose oracle: explicit element loops on small shapes, involution. CPU only."""

import numpy as np
import pytest

from oracle.transpose import transpose_i32
from thread_block_lds_amd import synth


@pytest.mark.parametrize("shape", [(1, 1), (1, 9), (9, 1), (3, 5), (64, 64), (17, 130)])
def test_transpose_elementwise(shape):
    x = synth.i32_uniform(shape, 7)
    y = transpose_i32(x)
    assert y.shape == (shape[1], shape[0]) and y.dtype == np.int32
    for i in range(shape[0]):
        for j in range(shape[1]):
            assert y[j, i] == x[i, j]
    assert np.array_equal(transpose_i32(y), x)
    assert y.flags["C_CONTIGUOUS"]
