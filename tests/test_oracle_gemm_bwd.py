"""Pins for the GEMM backward oracle (oracle/gemm_bwd.py): hand-worked products
and gradient casts, exact rational brute force, the transpose symmetry of the
two gradients, identity special cases, exact integer sums, and the positional
form against the full one."""
from fractions import Fraction

import numpy as np
import pytest

from oracle.gemm_bwd import cast_grad_f16, gemm_bwd, gemm_bwd_at
from tests.conftest import hexfloat, load_golden


def mat(rows, dtype):
    return np.array([[hexfloat(v) for v in r] for r in rows], dtype=dtype)


def test_golden_handworked():
    for case in load_golden("gemm_bwd_handworked.json")["cases"]:
        a, b = mat(case["a"], np.float16), mat(case["b"], np.float16)
        g = mat(case["g"], np.float32)
        (da, ta), (db, tb) = gemm_bwd(a, b, g)
        assert np.array_equal(da, mat(case["da"], np.float64))
        assert np.array_equal(db, mat(case["db"], np.float64))
        assert np.all(np.abs(da) <= ta) and np.all(np.abs(db) <= tb)


def test_cast_matches_ieee_half_conversion():
    # numpy's float32 -> float16 conversion is IEEE round-to-nearest-even
    rng = np.random.default_rng(12)
    g = (rng.standard_normal(20000) * np.exp2(rng.integers(-20, 16, 20000))).astype(np.float32)
    with np.errstate(over="ignore"):      # beyond 65504 both sides give +-inf
        ref = g.astype(np.float16).astype(np.float64)
    assert np.isinf(ref).any()
    assert np.array_equal(cast_grad_f16(g), ref)


def test_exact_rational_brute_force():
    rng = np.random.default_rng(13)
    m, n, k = 3, 17, 4
    a = rng.standard_normal((m, k)).astype(np.float16)
    b = rng.standard_normal((k, n)).astype(np.float16)
    g = rng.standard_normal((m, n)).astype(np.float32)
    g16 = g.astype(np.float16)
    (da, _), (db, _) = gemm_bwd(a, b, g)
    for i in range(m):
        for j in range(k):
            exact = sum(Fraction(float(g16[i, l])) * Fraction(float(b[j, l])) for l in range(n))
            assert abs(Fraction(da[i, j]) - exact) <= Fraction(1, 2 ** 40)
    for i in range(k):
        for j in range(n):
            exact = sum(Fraction(float(a[l, i])) * Fraction(float(g16[l, j])) for l in range(m))
            assert abs(Fraction(db[i, j]) - exact) <= Fraction(1, 2 ** 40)


def test_transpose_symmetry():
    # the backward of (B^T . A^T) with gradient G^T returns the transposed pair
    rng = np.random.default_rng(14)
    a = rng.standard_normal((9, 5)).astype(np.float16)
    b = rng.standard_normal((5, 7)).astype(np.float16)
    g = rng.standard_normal((9, 7)).astype(np.float32)
    (da, ta), (db, tb) = gemm_bwd(a, b, g)
    (da2, ta2), (db2, tb2) = gemm_bwd(np.ascontiguousarray(b.T), np.ascontiguousarray(a.T), np.ascontiguousarray(g.T))
    assert np.allclose(da2, db.T, rtol=0, atol=1e-12) and np.allclose(db2, da.T, rtol=0, atol=1e-12)
    assert np.allclose(ta2, tb.T, rtol=0, atol=1e-12) and np.allclose(tb2, ta.T, rtol=0, atol=1e-12)


def test_identities():
    rng = np.random.default_rng(15)
    g = rng.standard_normal((6, 8)).astype(np.float32)
    g16 = g.astype(np.float16).astype(np.float64)
    a = rng.standard_normal((6, 8)).astype(np.float16)
    (da, _), _ = gemm_bwd(a, np.eye(8, dtype=np.float16), g)
    assert np.array_equal(da, g16)
    b = rng.standard_normal((6, 8)).astype(np.float16)
    _, (db, _) = gemm_bwd(np.eye(6, dtype=np.float16), b, g)
    assert np.array_equal(db, g16)


def test_exact_integer_sums():
    rng = np.random.default_rng(16)
    m, n, k = 7, 300, 5
    ai = rng.integers(-8, 9, size=(m, k))
    bi = rng.integers(-8, 9, size=(k, n))
    gi = rng.integers(-8, 9, size=(m, n))
    (da, _), (db, _) = gemm_bwd(ai.astype(np.float16), bi.astype(np.float16), gi.astype(np.float32))
    assert np.array_equal(da, (gi @ bi.T).astype(np.float64))
    assert np.array_equal(db, (ai.T @ gi).astype(np.float64))


def test_positional_form_matches_full():
    rng = np.random.default_rng(17)
    a = rng.standard_normal((40, 24)).astype(np.float16)
    b = rng.standard_normal((24, 56)).astype(np.float16)
    g = rng.standard_normal((40, 56)).astype(np.float32)
    (da, ta), (db, tb) = gemm_bwd(a, b, g)
    ra, ca = rng.integers(0, 40, 500), rng.integers(0, 24, 500)
    rb, cb = rng.integers(0, 24, 500), rng.integers(0, 56, 500)
    (pa, pta), (pb, ptb) = gemm_bwd_at(a, b, g, ra, ca, rb, cb)
    assert np.allclose(pa, da[ra, ca], rtol=0, atol=1e-12) and np.allclose(pta, ta[ra, ca], rtol=0, atol=1e-12)
    assert np.allclose(pb, db[rb, cb], rtol=0, atol=1e-12) and np.allclose(ptb, tb[rb, cb], rtol=0, atol=1e-12)


def test_shape_checks():
    with pytest.raises(ValueError):
        gemm_bwd(np.zeros((2, 3), np.float16), np.zeros((4, 2), np.float16), np.zeros((2, 2), np.float32))
    with pytest.raises(ValueError):
        gemm_bwd(np.zeros((2, 3), np.float16), np.zeros((3, 2), np.float16), np.zeros((3, 2), np.float32))
