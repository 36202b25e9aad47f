"""INT8 packing convention -- oracle side (test infrastructure only).

Source: kaio-candle 0.2.0, src/qkv_project_int4.rs, module doc: the INT4
projection follows the same direct-call pattern as its W8A16 sibling
``qkv_project_int8``.  That sibling's weight layout is not printed on the
pages; this library reads it as the 8-bit analogue of the INT4 packing
(stated once, used everywhere):

* ``u32[K/4, N]``: four INT8 values per 32-bit word, packed along K;
* signed two's complement, values in [-128, 127], no zero point;
* byte i of a word (bits 8i .. 8i+7, least significant byte first) of packed
  row r, column n holds the weight at reduction index k = 4*r + i, column n;
* the packed tensor is row-major, so word (r, n) sits at offset r*N + n.
"""
from __future__ import annotations

import numpy as np


def unpack_int8(words: np.ndarray) -> np.ndarray:
    """u32[R, N] -> int16[4R, N]; row 4r+i of the result is byte i of packed row r."""
    words = np.asarray(words)
    if words.dtype != np.uint32 or words.ndim != 2:
        raise ValueError("packed weights must be a 2-D uint32 array")
    R, N = words.shape
    q = np.empty((4 * R, N), dtype=np.int16)
    w64 = words.astype(np.int64)
    for i in range(4):
        byte = (w64 >> (8 * i)) & 0xFF
        q[i::4, :] = np.where(byte >= 128, byte - 256, byte)
    return q


def pack_int8(q: np.ndarray) -> np.ndarray:
    """int[4R, N] with values in [-128, 127] -> u32[R, N] (inverse of ``unpack_int8``)."""
    q = np.asarray(q)
    if q.ndim != 2 or q.shape[0] % 4:
        raise ValueError("q must be 2-D with a multiple of 4 rows")
    if q.size and (q.min() < -128 or q.max() > 127):
        raise ValueError("INT8 values must lie in [-128, 127]")
    R = q.shape[0] // 4
    words = np.zeros((R, q.shape[1]), dtype=np.int64)
    for i in range(4):
        words |= (q[i::4, :].astype(np.int64) & 0xFF) << (8 * i)
    return words.astype(np.uint32)
