"""Backward of the dense f16 x f16 -> f32 matmul -- oracle side (test infrastructure only).

Source: kaio-candle 0.2.0, src/matmul_tc_async.rs -- ``MatmulTcAsyncOp::bwd``:
the f32 output gradient is cast to f16, then dA = grad . B^T and
dB = A^T . grad are formed by the forward kernel (f16 x f16 -> f32) and each
f32 result is cast to f16.

    G16[i, l]  = RNE_f16(G[i, l])
    dA*[i, j]  = sum_l G16[i, l] * B[j, l]          A: [m, k]  B: [k, n]  G: [m, n]
    dB*[i, j]  = sum_l A[l, i] * G16[l, j]
    T_A, T_B   = the same sums of |products|        (for the tolerance)

Everything in float64 (f16 x f16 products are exact).  The GPU result is an
f32 accumulation rounded once to f16, compared with the tolerance of an f16
output: |d - Y*| <= ulp16(Y*) + 1e-5 * T.
"""
from __future__ import annotations

import numpy as np

from .rounding import round_to_format


def cast_grad_f16(g) -> np.ndarray:
    """The f16 rounding (nearest even) of an f32 gradient, as float64 values."""
    return round_to_format(np.asarray(g, dtype=np.float64), "f16")


def gemm_bwd(a, b, g, with_abs=True):
    """((dA*, T_A), (dB*, T_B)) for A f16[m,k], B f16[k,n], G f32[m,n]."""
    a = np.asarray(a)
    b = np.asarray(b)
    g = np.asarray(g)
    if a.ndim != 2 or b.ndim != 2 or g.ndim != 2:
        raise ValueError("a, b and g must be matrices")
    m, k = a.shape
    if b.shape[0] != k or g.shape != (m, b.shape[1]):
        raise ValueError(f"shape mismatch: a {a.shape}, b {b.shape}, g {g.shape}")
    a64 = a.astype(np.float64)
    b64 = b.astype(np.float64)
    g16 = cast_grad_f16(g)
    da = g16 @ b64.T
    db = a64.T @ g16
    if not with_abs:
        return (da, None), (db, None)
    ta = np.abs(g16) @ np.abs(b64).T
    tb = np.abs(a64).T @ np.abs(g16)
    return (da, ta), (db, tb)


def gemm_bwd_at(a, b, g, rows_a, cols_a, rows_b, cols_b):
    """dA*, T_A at the positions (rows_a[i], cols_a[i]) and dB*, T_B at (rows_b[i], cols_b[i])."""
    a = np.asarray(a).astype(np.float64)
    b = np.asarray(b).astype(np.float64)
    g16 = cast_grad_f16(g)
    pa = g16[np.asarray(rows_a)] * b[np.asarray(cols_a)]            # [P, n] products
    pb = a[:, np.asarray(rows_b)].T * g16[:, np.asarray(cols_b)].T   # [P, m] products
    return (pa.sum(axis=1), np.abs(pa).sum(axis=1)), (pb.sum(axis=1), np.abs(pb).sum(axis=1))
