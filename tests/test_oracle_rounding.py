"""Pins for the oracle's round-to-nearest-even (oracle/rounding.py).

Hand-worked halfway and overflow cases (tests/golden/rounding_cases.json),
plus agreement with rounding routines the oracle does not call: numpy's
float64 -> float32 / float16 casts and torch's float32 -> bfloat16 cast.
"""
import numpy as np
import torch

from oracle.rounding import (bf16_bits_to_f64, f64_to_bf16_bits, round_to_format)
from tests.conftest import hexfloat, load_golden


def test_golden_cases():
    for fmt, v, expect in load_golden("rounding_cases.json")["cases"]:
        got = round_to_format(np.array([hexfloat(v)]), fmt)[0]
        assert got == hexfloat(expect) and np.signbit(got) == np.signbit(hexfloat(expect)), (fmt, v, expect, got)


def _random_f64(n, seed, lo, hi):
    rng = np.random.default_rng(seed)
    mant = rng.random(n) + 0.5
    exps = rng.integers(lo, hi, size=n)
    sign = np.where(rng.random(n) < 0.5, -1.0, 1.0)
    return sign * np.ldexp(mant, exps)


def test_matches_numpy_float32_cast():
    v = _random_f64(400_000, 1, -160, 130)
    # values exactly halfway between two float32 neighbours
    f = _random_f64(50_000, 2, -120, 120).astype(np.float32).astype(np.float64)
    ties = f + np.spacing(f.astype(np.float32)).astype(np.float64) / 2
    for arr in (v, ties):
        with np.errstate(over="ignore"):
            ref = arr.astype(np.float32).astype(np.float64)
        got = round_to_format(arr, "f32")
        assert np.array_equal(got, ref)


def test_matches_numpy_float16_cast():
    v = _random_f64(400_000, 3, -30, 18)
    f = _random_f64(50_000, 4, -24, 15).astype(np.float16)
    ties = f.astype(np.float64) + np.spacing(f).astype(np.float64) / 2
    for arr in (v, ties):
        with np.errstate(over="ignore"):
            ref = arr.astype(np.float16).astype(np.float64)
        got = round_to_format(arr, "f16")
        assert np.array_equal(got, ref)


def test_matches_torch_bfloat16_cast():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2 ** 32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    f32 = bits.view(np.float32)
    f32 = f32[np.isfinite(f32)]
    ref = torch.from_numpy(f32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = f64_to_bf16_bits(f32.astype(np.float64))
    assert np.array_equal(got, ref)
    # and the widening is exact
    back = bf16_bits_to_f64(got)
    ref_back = torch.from_numpy(ref.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    assert np.array_equal(back, ref_back.astype(np.float64))


def test_special_values_pass_through():
    v = np.array([0.0, -0.0, np.inf, -np.inf, np.nan])
    for fmt in ("f32", "bf16", "f16"):
        got = round_to_format(v, fmt)
        assert got[0] == 0 and not np.signbit(got[0])
        assert got[1] == 0 and np.signbit(got[1])
        assert got[2] == np.inf and got[3] == -np.inf and np.isnan(got[4])
