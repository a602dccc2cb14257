"""Group-quantized weights: the dequantization the quantized weight product computes
(test infrastructure only: the tests, the smoke check and the benchmark's CPU baseline use it).

[W] §4.2 describes group quantization: a weight matrix stored as integers, split into groups (for
example 128 consecutive elements), each group carrying one scale and one zero point; before the
matrix product the integers are turned back into floating point through the scales.  The page gives
no formula; the reading taken is the usual asymmetric one, value = (code - zero) * scale, with 8-bit
unsigned codes and zero points and the groups running along each row (the input dimension of an
[out][in] matrix).  A row whose length is not a multiple of the group size ends with one shorter
group (the page gives 128 as an example size and says nothing of rows that do not divide); it has
its own scale and zero point like any other.

The page names int4 as well as int8 codes.  4-bit codes travel two to a byte, the even column in the
low nibble and the odd column in the high nibble (the storage convention of the library's interface);
unpack_nibbles turns such rows back into one code per column.
"""
from __future__ import annotations

import numpy as np

GROUP = 128


def dequantize(codes, scales, zeros, group: int = GROUP) -> np.ndarray:
    """codes [rows][cols] uint8, scales and zeros [rows][ceil(cols/group)] -> float64 [rows][cols] with
    w[r, c] = (codes[r, c] - zeros[r, c // group]) * scales[r, c // group]."""
    codes = np.asarray(codes)
    rows, cols = codes.shape
    g = (cols + group - 1) // group
    z = np.asarray(zeros, dtype=np.float64)
    s = np.asarray(scales, dtype=np.float64)
    assert z.shape == (rows, g) and s.shape == (rows, g), "one scale and one zero point per group"
    col_group = np.arange(cols) // group            # the group of every column
    return (codes.astype(np.float64) - z[:, col_group]) * s[:, col_group]


def linear_q8(x, codes, scales, zeros) -> np.ndarray:
    """y = x W^T with W the dequantized [out][in] matrix, in float64."""
    return np.asarray(x, dtype=np.float64) @ dequantize(codes, scales, zeros).T


def unpack_nibbles(packed, cols: int) -> np.ndarray:
    """packed [rows][cols/2] uint8, two 4-bit codes per byte (column 2j in the low nibble of byte j, 2j+1
    in the high nibble) -> codes [rows][cols] uint8 in 0..15."""
    packed = np.asarray(packed, dtype=np.uint8)
    rows = packed.shape[0]
    out = np.empty((rows, cols), np.uint8)
    out[:, 0::2] = packed[:, : (cols + 1) // 2] & 0x0F
    out[:, 1::2] = packed[:, : cols // 2] >> 4
    return out
