"""Dense f16 x f16 -> f32 matmul -- oracle side (test infrastructure only).

Source: kaio-candle 0.2.0, src/matmul_tc_async.rs -- module doc (f16 x f16
-> f32 matmul) and ``MatmulTcAsyncOp::cuda_fwd`` (A ``[m, k]``, B ``[k, n]``,
inner dimensions must match, the output ``[m, n]`` f32 is freshly zeroed and
then written, so the result is C = A.B with no accumulation into C).

    C[i, j] = sum_k A[i, k] * B[k, j]        (float64; f16 products are exact)
    T[i, j] = sum_k |A[i, k] * B[k, j]|      (for the tolerance)
"""
from __future__ import annotations

import numpy as np


def gemm(a, b, with_abs=True):
    a = np.asarray(a)
    b = np.asarray(b)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[0]:
        raise ValueError(f"K mismatch: A {a.shape}, B {b.shape}")
    a64 = a.astype(np.float64)
    b64 = b.astype(np.float64)
    c = a64 @ b64
    t = np.abs(a64) @ np.abs(b64) if with_abs else None
    return c, t


def gemm_at(a, b, rows, cols):
    """C and T at the listed (rows[i], cols[i]) positions only."""
    a = np.asarray(a)
    b = np.asarray(b)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[0]:
        raise ValueError(f"K mismatch: A {a.shape}, B {b.shape}")
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    c = np.empty(rows.shape[0])
    t = np.empty(rows.shape[0])
    step = 1024
    for lo in range(0, rows.shape[0], step):
        ar = a[rows[lo:lo + step]].astype(np.float64)
        bc = b[:, cols[lo:lo + step]].astype(np.float64).T
        prod = ar * bc
        c[lo:lo + step] = prod.sum(axis=1)
        t[lo:lo + step] = np.abs(prod).sum(axis=1)
    return c, t
