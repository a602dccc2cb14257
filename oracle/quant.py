"""Group-quantized weights: the dequantization the quantized weight product computes
(test infrastructure only: the tests, the smoke check and the benchmark's CPU baseline use it).

[W] §4.2 describes group quantization: a weight matrix stored as integers, split into groups (for
example 128 consecutive elements), each group carrying one scale and one zero point; before the
matrix product the integers are turned back into floating point through the scales.  The page gives
no formula; the reading taken is the usual asymmetric one, value = (code - zero) * scale, with 8-bit
unsigned codes and zero points and the groups running along each row (the input dimension of an
[out][in] matrix).
"""
from __future__ import annotations

import numpy as np

GROUP = 128


def dequantize(codes, scales, zeros, group: int = GROUP) -> np.ndarray:
    """codes [rows][cols] uint8, scales [rows][cols/group] float, zeros [rows][cols/group] uint8 ->
    float64 [rows][cols] with w[r, c] = (codes[r, c] - zeros[r, c // group]) * scales[r, c // group]."""
    codes = np.asarray(codes)
    rows, cols = codes.shape
    assert cols % group == 0, "cols must be a whole number of groups"
    g = cols // group
    q = codes.astype(np.float64).reshape(rows, g, group)
    z = np.asarray(zeros, dtype=np.float64).reshape(rows, g, 1)
    s = np.asarray(scales, dtype=np.float64).reshape(rows, g, 1)
    return ((q - z) * s).reshape(rows, cols)


def linear_q8(x, codes, scales, zeros) -> np.ndarray:
    """y = x W^T with W the dequantized [out][in] matrix, in float64."""
    return np.asarray(x, dtype=np.float64) @ dequantize(codes, scales, zeros).T
