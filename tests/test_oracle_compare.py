"""Pins for the parity tolerances (oracle/compare.py)."""
import numpy as np

from oracle.compare import bits_equal, excess, qkv_tolerance, ulp16


def test_ulp16_hand_values():
    v = np.array([1.0, 1.5, 1.999, 2.0, 65504.0, 2.0 ** -14, 2.0 ** -15, 0.0, -3.0, 1e-9])
    want = np.array([2.0 ** -10, 2.0 ** -10, 2.0 ** -10, 2.0 ** -9, 32.0, 2.0 ** -24,
                     2.0 ** -24, 2.0 ** -24, 2.0 ** -9, 2.0 ** -24])
    assert np.array_equal(ulp16(v), want)


def test_ulp16_is_numpy_spacing_on_f16_values():
    f = np.arange(0, 0x7BFF, dtype=np.uint16).view(np.float16)      # every finite non-negative f16 below the largest
    assert np.array_equal(ulp16(f.astype(np.float64)), np.spacing(f).astype(np.float64))


def test_excess_and_bits():
    ref = np.array([1.0, 2.0])
    tol = qkv_tolerance(ref, np.array([0.0, 0.0]))
    assert excess(np.array([1.0 + 2.0 ** -10, 2.0]), ref, tol) == (0, 1.0)
    n, r = excess(np.array([1.0 + 2.0 ** -9, np.nan]), ref, tol)
    assert n == 2 and r == np.inf
    a = np.array([1.0, np.nan, -0.0], dtype=np.float32)
    b = np.array([1.0, np.nan, 0.0], dtype=np.float32)
    assert bits_equal(a, b).tolist() == [True, True, False]
