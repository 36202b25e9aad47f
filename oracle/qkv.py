"""W4A16 fused tri-output QKV projection -- oracle side (test infrastructure only).

Source: kaio-candle 0.2.0, src/qkv_project_int4.rs -- the module doc (one
launch, seven inputs, ``group_size`` fixed at 128, K a multiple of 128), the
doc comment of ``qkv_project_int4`` (x ``f16[M,K]``; packed weights
``u32[K/8,N]``; scales ``f16[K/128,N]``, one per group of 128 along K;
outputs three ``f16[M,N]``) and its validation chain (K multiple of 128,
packed rows K/8, scale rows K/128, one N for all six weight/scale tensors).

For each projection p in (q, k, v):

    w_p[k, n] = int4(W_p, k, n) * S_p[k // 128, n]          (exact in float64)
    Y_p[m, n] = sum_k x[m, k] * w_p[k, n]                   (float64)
    T_p[m, n] = sum_k |x[m, k] * w_p[k, n]|                 (for the tolerance)

``Y_p`` is returned unrounded; the GPU's f16 output is judged against it with
the tolerance in ``compare``.  The f64 matmul (a library primitive) forms the
sums; every product q*s and x*w is exact in float64 (<= 4+11+11 significant
bits), so only the summation order differs from the plain loop.

The W8A16 sibling (``bits=8``) is the same definition with INT8 weights
``u32[K/4, N]`` decoded by ``oracle.int8`` (its layout is a reading: see that
module); every product q*s (<= 8+11 significant bits) and x*w is still exact
in float64.
"""
from __future__ import annotations

import numpy as np

from .int4 import unpack_int4
from .int8 import unpack_int8

GROUP_SIZE = 128
UNPACK = {4: unpack_int4, 8: unpack_int8}


def packed_rows(K: int, bits: int) -> int:
    """Rows of the packed weight tensor: K / (32 / bits) values per column, 32/bits per word."""
    return K * bits // 32


def dequantize(words: np.ndarray, scales: np.ndarray, bits: int = 4) -> np.ndarray:
    """u32[K*bits/32, N] and f16[K/128, N] -> float64 w[K, N] = q * scale[k // 128, n]."""
    q = UNPACK[bits](words).astype(np.float64)
    K, N = q.shape
    s = np.asarray(scales)
    if s.shape != (K // GROUP_SIZE, N):
        raise ValueError(f"scales must be [K/128, N] = [{K // GROUP_SIZE}, {N}], got {s.shape}")
    group_of_k = np.arange(K) // GROUP_SIZE
    return q * s.astype(np.float64)[group_of_k, :]


def check_shapes(x, w, s, bits=4):
    x = np.asarray(x)
    if x.ndim != 2:
        raise ValueError("x must be [M, K]")
    M, K = x.shape
    if K % GROUP_SIZE:
        raise ValueError(f"K ({K}) must be a multiple of group_size ({GROUP_SIZE})")
    if len(w) != 3 or len(s) != 3:
        raise ValueError("need three packed weights and three scale tensors")
    N = np.asarray(w[0]).shape[1]
    for wp in w:
        if np.asarray(wp).shape != (packed_rows(K, bits), N):
            raise ValueError(f"packed weights must be [K*{bits}/32, N] = [{packed_rows(K, bits)}, {N}]")
    for sp in s:
        if np.asarray(sp).shape != (K // GROUP_SIZE, N):
            raise ValueError(f"scales must be [K/128, N] = [{K // GROUP_SIZE}, {N}]")
    return M, N, K


def qkv_project(x, w, s, rows=None, with_abs=True, bits=4):
    """Returns ([Y_q, Y_k, Y_v], [T_q, T_k, T_v]) in float64.

    ``bits`` is the weight width: 4 (W4A16, ``u32[K/8, N]``) or 8 (W8A16,
    ``u32[K/4, N]``).

    ``rows`` optionally selects a subset of the rows of x (same definition,
    fewer outputs) so that full-size problems can be checked on a sample.
    """
    if bits not in UNPACK:
        raise ValueError(f"bits must be 4 or 8, got {bits}")
    M, N, K = check_shapes(x, w, s, bits)
    x64 = np.asarray(x).astype(np.float64)
    if rows is not None:
        x64 = x64[np.asarray(rows)]
    ys, ts = [], []
    for wp, sp in zip(w, s):
        wd = dequantize(np.asarray(wp), np.asarray(sp), bits)
        ys.append(x64 @ wd)
        ts.append(np.abs(x64) @ np.abs(wd) if with_abs else None)
    return ys, ts
