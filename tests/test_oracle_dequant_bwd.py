"""Pins for the dequant-backward oracle (oracle/dequant_bwd.py): hand-worked
products and ties (tests/golden/dequant_bwd_handworked.json), exact rational
products, the group index, and the plan's problem checks."""
from fractions import Fraction

import numpy as np
import pytest

from oracle.dequant_bwd import DTYPES, dequant_bwd
from oracle.rounding import f64_to_storage, storage_to_f64
from tests.conftest import hexfloat, load_golden


def to_storage(vals, dtype):
    arr = np.array([[hexfloat(v) for v in row] for row in vals], dtype=np.float64)
    st = f64_to_storage(arr, dtype)
    assert np.array_equal(storage_to_f64(st, dtype), arr), "fixture values must be exact in the dtype"
    return st


def test_golden_handworked():
    for case in load_golden("dequant_bwd_handworked.json")["cases"]:
        for dt in case["dtypes"]:
            dy = to_storage(case["dy"], dt)
            sc = to_storage(case["scale"], dt)
            got = storage_to_f64(dequant_bwd(dy, sc, case["group"], dt), dt)
            want = np.array([[hexfloat(v) for v in row] for row in case["dq"]])
            assert np.array_equal(got, want), (case["name"], dt, got, want)


def _all_values(dtype):
    """Every finite value of a 16-bit format with its bit pattern, sorted by value."""
    bits = np.arange(0, 2 ** 16, dtype=np.uint32).astype(np.uint16)
    if dtype == "f16":
        vals = bits.view(np.float16).astype(np.float64)
    else:
        with np.errstate(invalid="ignore"):
            vals = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    keep = np.isfinite(vals) & ~((vals == 0) & (bits != 0))
    order = np.argsort(vals[keep], kind="stable")
    return vals[keep][order], bits[keep][order]


def _nearest_even(exact, vals, bits):
    i = int(np.searchsorted(vals, float(exact)))
    cands = [j for j in (i - 1, i, i + 1) if 0 <= j < len(vals)]
    dist = [abs(Fraction(float(vals[j])) - exact) for j in cands]
    best = min(dist)
    ties = [cands[k] for k in range(len(cands)) if dist[k] == best]
    return [float(vals[j]) for j in ties if int(bits[j]) % 2 == 0] or [float(vals[ties[0]])]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_exact_rational_then_nearest(dtype):
    """dq is the format value nearest the exact rational product, ties to the even pattern.
    The neighbours come from enumerating the format (16-bit) or float32 nextafter, not from
    the oracle's rounding routine."""
    from int4_group_quantized_w4a16_amd.workloads import dequant_bwd_inputs
    dy, sc = dequant_bwd_inputs(3, 48, 16, 9, dtype)
    dq = storage_to_f64(dequant_bwd(dy, sc, 16, dtype), dtype)
    dy64 = storage_to_f64(dy, dtype)
    sc64 = storage_to_f64(sc, dtype)
    table = _all_values(dtype) if dtype != "f32" else None
    for i in range(3):
        for j in range(48):
            exact = Fraction(float(dy64[i, j])) * Fraction(float(sc64[i, j // 16]))
            if table is not None:
                assert float(dq[i, j]) in _nearest_even(exact, *table)
            else:
                r = np.float32(dq[i, j])
                lo = np.nextafter(r, np.float32(-np.inf))
                hi = np.nextafter(r, np.float32(np.inf))
                d = abs(Fraction(float(r)) - exact)
                assert d <= abs(Fraction(float(lo)) - exact) and d <= abs(Fraction(float(hi)) - exact)


def test_f64_is_the_ieee_product():
    rng = np.random.default_rng(10)
    dy = rng.standard_normal((4, 12))
    sc = rng.uniform(0.001, 0.1, size=(4, 3))
    dq = dequant_bwd(dy, sc, 4, "f64")
    for i in range(4):
        for j in range(12):
            assert dq[i, j] == float(dy[i, j]) * float(sc[i, j // 4])


def test_group_index():
    # scale column g is the power of two 2**g, so dq / dy reads the group back
    outer, axis, g = 2, 40, 8
    dy = np.ones((outer, axis), dtype=np.float32)
    sc = np.stack([2.0 ** np.arange(axis // g), 2.0 ** -np.arange(axis // g)]).astype(np.float32)
    dq = dequant_bwd(dy, sc, g, "f32")
    j = np.arange(axis)
    assert np.array_equal(dq[0], 2.0 ** (j // g))
    assert np.array_equal(dq[1], 2.0 ** -(j // g))


def test_unit_scale_is_identity_and_problem_checks():
    for dt in DTYPES:
        from int4_group_quantized_w4a16_amd.workloads import dequant_bwd_inputs
        dy, _ = dequant_bwd_inputs(2, 8, 4, 1, dt)
        one = f64_to_storage(np.ones((2, 2)), dt)
        assert np.array_equal(dequant_bwd(dy, one, 4, dt), dy)
    ok = np.zeros((1, 4), np.float32)
    with pytest.raises(ValueError):
        dequant_bwd(ok, np.zeros((1, 1), np.float32), 3, "f32")     # axis % group
    with pytest.raises(ValueError):
        dequant_bwd(ok, np.zeros((1, 1), np.float32), 0, "f32")     # group <= 0
    with pytest.raises(ValueError):
        dequant_bwd(ok, np.zeros((1, 2), np.float32), 4, "f32")     # scale shape
    with pytest.raises(ValueError):
        dequant_bwd(ok, np.zeros((1, 1), np.float32), 4, "s8")      # dtype
    empty = dequant_bwd(np.zeros((0, 8), np.float32), np.zeros((0, 2), np.float32), 4, "f32")
    assert empty.shape == (0, 8)
