"""Round-to-nearest-even into a narrow binary format -- oracle side (test infrastructure only).

Written from the IEEE-754 definition: a finite binary format with ``p``
significand bits and minimum normal exponent ``emin`` has, at magnitude
|v| in [2^e, 2^(e+1)), a spacing of 2^(e-p+1) (and 2^(emin-p+1) below 2^emin,
the subnormal range).  Rounding picks the nearest multiple of that spacing,
ties to the even multiple; magnitudes beyond the largest finite value after
rounding become infinity.

Used for the single rounded multiply of the dequant backward (baracuda-kernels
0.0.1-alpha.68, src/quantize/dequantize_per_group_backward.rs: the plan's
"deterministic, bit-stable" precision guarantee) and to read/write bf16 bit
patterns, which numpy lacks.
"""
from __future__ import annotations

import numpy as np

# (significand bits p, emin, emax)
FORMATS = {
    "f64": (53, -1022, 1023),
    "f32": (24, -126, 127),
    "bf16": (8, -126, 127),
    "f16": (11, -14, 15),
}


def round_to_format(v: np.ndarray, fmt: str) -> np.ndarray:
    """Round float64 values to the nearest value of ``fmt`` (ties to even); returns float64."""
    p, emin, emax = FORMATS[fmt]
    v = np.asarray(v, dtype=np.float64)
    out = v.copy()
    finite = np.isfinite(v) & (v != 0)
    a = np.abs(v[finite])
    _, E = np.frexp(a)                    # a = m * 2**E with m in [0.5, 1)
    e = np.maximum(E - 1, emin)           # floor(log2 a), clamped into the subnormal binade
    spacing = np.ldexp(1.0, e - (p - 1))
    r = np.rint(v[finite] / spacing) * spacing   # the division by a power of two is exact
    largest = np.ldexp(2.0 - np.ldexp(1.0, 1 - p), emax)
    r = np.where(np.abs(r) > largest, np.copysign(np.inf, r), r)
    out[finite] = r
    return out


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 is the upper half of an IEEE binary32 word."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 (RNE, once) and return the 16-bit patterns."""
    r = round_to_format(v, "bf16").astype(np.float32)   # exact: every bf16 value is an f32
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def storage_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored values (bf16 given as uint16 patterns)."""
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    return np.asarray(a).astype(np.float64)


def f64_to_storage(v: np.ndarray, dtype: str) -> np.ndarray:
    """Single RNE rounding of float64 values to the storage dtype."""
    if dtype == "bf16":
        return f64_to_bf16_bits(v)
    if dtype == "f64":
        return np.asarray(v, dtype=np.float64).copy()
    r = round_to_format(v, dtype)
    return r.astype(np.float32 if dtype == "f32" else np.float16)  # exact after rounding
