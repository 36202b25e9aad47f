"""Parity tolerances -- oracle side (test infrastructure only).

* f32 GEMM outputs:   |d| <= 1e-5 * T,                    T = sum_k |a_ik * b_kj|
* f16 Q/K/V outputs:  |d| <= ulp16(Y*) + 1e-5 * T,        T = sum_k |x_ik * w_kj|
  (the same bound for the f16 gradients of the GEMM backward, T = sum |products|)
* dequant backward:   bit-exact (one rounded multiply per element).

``Y*`` is the unrounded float64 oracle value.  ``ulp16(v)`` is the spacing of
IEEE binary16 at v: 2**(floor(log2|v|) - 10) for |v| >= 2**-14 (normal
range) and 2**-24 below it (subnormal range, including v = 0).  The f16
output is itself a rounding of an f32 accumulator, which is what the one-ulp
term allows for; the 1e-5 * T term bounds the f32 accumulation error.
"""
from __future__ import annotations

import numpy as np

QKV_REL = 1e-5
GEMM_REL = 1e-5


def ulp16(v: np.ndarray) -> np.ndarray:
    a = np.abs(np.asarray(v, dtype=np.float64))
    _, E = np.frexp(a)                      # a = m * 2**E, m in [0.5, 1)
    e = np.maximum(E - 1, -14)              # floor(log2 a), clamped to the subnormal binade
    return np.where(a >= 2.0 ** -14, np.ldexp(1.0, e - 10), 2.0 ** -24)


def qkv_tolerance(y_ref, t_ref):
    return ulp16(y_ref) + QKV_REL * np.asarray(t_ref, dtype=np.float64)


def f16_tolerance(y_ref, t_ref):
    """Any f16 output of an f32 accumulation: one f16 ulp plus the accumulation bound."""
    return qkv_tolerance(y_ref, t_ref)


def gemm_tolerance(t_ref):
    return GEMM_REL * np.asarray(t_ref, dtype=np.float64)


def excess(got, ref, tol):
    """(number of violations, max |got - ref| / tol); NaN/inf in ``got`` count as violations."""
    got = np.asarray(got, dtype=np.float64)
    d = np.abs(got - np.asarray(ref, dtype=np.float64))
    bad = ~np.isfinite(d) | (d > tol)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(np.isfinite(d), d / tol, np.inf)
    return int(bad.sum()), float(ratio.max()) if ratio.size else 0.0


def bits_equal(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Element-wise bit equality, with every NaN equal to every NaN."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    if got.dtype != ref.dtype or got.shape != ref.shape:
        raise ValueError(f"dtype/shape mismatch: {got.dtype}{got.shape} vs {ref.dtype}{ref.shape}")
    if got.dtype == np.uint16:           # bf16 patterns
        g = got.astype(np.uint32) << 16
        r = ref.astype(np.uint32) << 16
        gn = np.isnan(g.view(np.float32))
        rn = np.isnan(r.view(np.float32))
        return (got == ref) | (gn & rn)
    view = {2: np.uint16, 4: np.uint32, 8: np.uint64}[got.dtype.itemsize]
    eq = got.view(view) == ref.view(view)
    return eq | (np.isnan(got) & np.isnan(ref))
