"""INT4 packing convention -- oracle side (test infrastructure only).

Source: kaio-candle 0.2.0, src/qkv_project_int4.rs, doc comment of
``qkv_project_int4``: each packed weight tensor is ``u32[K/8, N]`` with eight
INT4 values per 32-bit word.  The page does not fix signedness or nibble
order; this library reads them as follows (stated once, used everywhere):

* signed two's complement, values in [-8, 7], no zero point;
* nibble i of a word (bits 4i .. 4i+3, least significant nibble first) of
  packed row r, column n holds the weight at reduction index k = 8*r + i,
  column n;
* the packed tensor is row-major, so word (r, n) sits at offset r*N + n.
"""
from __future__ import annotations

import numpy as np


def unpack_int4(words: np.ndarray) -> np.ndarray:
    """u32[R, N] -> int8[8R, N]; row 8r+i of the result is nibble i of packed row r."""
    words = np.asarray(words)
    if words.dtype != np.uint32 or words.ndim != 2:
        raise ValueError("packed weights must be a 2-D uint32 array")
    R, N = words.shape
    q = np.empty((8 * R, N), dtype=np.int8)
    w64 = words.astype(np.int64)
    for i in range(8):
        nib = (w64 >> (4 * i)) & 0xF
        q[i::8, :] = np.where(nib >= 8, nib - 16, nib)
    return q


def pack_int4(q: np.ndarray) -> np.ndarray:
    """int[8R, N] with values in [-8, 7] -> u32[R, N] (inverse of ``unpack_int4``)."""
    q = np.asarray(q)
    if q.ndim != 2 or q.shape[0] % 8:
        raise ValueError("q must be 2-D with a multiple of 8 rows")
    if q.size and (q.min() < -8 or q.max() > 7):
        raise ValueError("INT4 values must lie in [-8, 7]")
    R = q.shape[0] // 8
    words = np.zeros((R, q.shape[1]), dtype=np.int64)
    for i in range(8):
        words |= (q[i::8, :].astype(np.int64) & 0xF) << (4 * i)
    return words.astype(np.uint32)
