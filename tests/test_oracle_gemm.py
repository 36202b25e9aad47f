"""Pins for the dense GEMM oracle (oracle/gemm.py): hand-worked products,
identity, exact integer products, and agreement between the full and the
positional forms."""
import numpy as np
import pytest

from oracle.gemm import gemm, gemm_at
from tests.conftest import load_golden


def test_golden_handworked():
    for case in load_golden("gemm_handworked.json")["cases"]:
        a = np.array(case["a"], dtype=np.float16)
        b = np.array(case["b"], dtype=np.float16)
        c, t = gemm(a, b)
        assert np.array_equal(c, np.array(case["c"], dtype=np.float64))
        assert np.all(np.abs(c) <= t)


def test_identity():
    rng = np.random.default_rng(3)
    a = rng.standard_normal((64, 96)).astype(np.float16)
    c, _ = gemm(a, np.eye(96, dtype=np.float16))
    assert np.array_equal(c, a.astype(np.float64))
    c, _ = gemm(np.eye(64, dtype=np.float16), a)
    assert np.array_equal(c, a.astype(np.float64))


def test_exact_integer_products_against_python_ints():
    rng = np.random.default_rng(4)
    M, N, K = 9, 7, 300
    ai = rng.integers(-8, 9, size=(M, K))
    bi = rng.integers(-8, 9, size=(K, N))
    c, t = gemm(ai.astype(np.float16), bi.astype(np.float16))
    for i in range(M):
        for j in range(N):
            exact = sum(int(ai[i, k]) * int(bi[k, j]) for k in range(K))
            exact_abs = sum(abs(int(ai[i, k]) * int(bi[k, j])) for k in range(K))
            assert c[i, j] == exact and t[i, j] == exact_abs


def test_exact_dyadic_brute_force():
    from fractions import Fraction
    rng = np.random.default_rng(6)
    a = rng.standard_normal((4, 33)).astype(np.float16)
    b = rng.standard_normal((33, 5)).astype(np.float16)
    c, _ = gemm(a, b)
    for i in range(4):
        for j in range(5):
            exact = sum(Fraction(float(a[i, k])) * Fraction(float(b[k, j])) for k in range(33))
            assert abs(Fraction(c[i, j]) - exact) <= Fraction(1, 2 ** 40)


def test_positional_form_matches_full():
    rng = np.random.default_rng(8)
    a = rng.standard_normal((40, 64)).astype(np.float16)
    b = rng.standard_normal((64, 50)).astype(np.float16)
    c, t = gemm(a, b)
    rows = rng.integers(0, 40, size=3000)
    cols = rng.integers(0, 50, size=3000)
    cp, tp = gemm_at(a, b, rows, cols)
    assert np.allclose(cp, c[rows, cols], rtol=0, atol=1e-12)
    assert np.allclose(tp, t[rows, cols], rtol=0, atol=1e-12)


def test_k_mismatch_and_empty():
    with pytest.raises(ValueError):
        gemm(np.zeros((2, 3), np.float16), np.zeros((4, 2), np.float16))
    c, t = gemm(np.zeros((3, 0), np.float16), np.zeros((0, 2), np.float16))
    assert c.shape == (3, 2) and not c.any()
