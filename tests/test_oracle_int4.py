"""Pins for the oracle's INT4 decoding (oracle/int4.py).

The convention (signed, low nibble first, k = 8r + i) is read off hex digits
here -- digit i counted from the right of the word's 8-digit hex string -- a
route that shares nothing with the oracle's shift-and-mask decoder.
"""
import numpy as np
import pytest

from oracle.int4 import pack_int4, unpack_int4
from tests.conftest import load_golden


def hex_decode(word):
    digits = format(int(word), "08x")
    vals = [int(digits[7 - i], 16) for i in range(8)]
    return [v - 16 if v >= 8 else v for v in vals]


def test_golden_words():
    for case in load_golden("int4_words.json")["cases"]:
        word = int(case["word"], 16)
        q = np.array(case["q"], dtype=np.int64).reshape(8, 1)
        assert int(pack_int4(q)[0, 0]) == word, case
        assert unpack_int4(np.array([[word]], dtype=np.uint32))[:, 0].tolist() == case["q"]
        assert hex_decode(word) == case["q"]


def test_every_nibble_position_and_value():
    # 8 positions x 16 values, words built from hex strings (no shifts).
    for i in range(8):
        for v in range(16):
            digits = ["0"] * 8
            digits[7 - i] = format(v, "x")
            word = int("".join(digits), 16)
            q = unpack_int4(np.array([[word]], dtype=np.uint32))[:, 0]
            expect = np.zeros(8, dtype=np.int64)
            expect[i] = v - 16 if v >= 8 else v
            assert q.tolist() == expect.tolist(), (i, v)


def test_layout_rows_and_columns():
    rng = np.random.default_rng(7)
    words = rng.integers(0, 2 ** 32, size=(5, 3), dtype=np.uint32)
    q = unpack_int4(words)
    assert q.shape == (40, 3)
    for r in range(5):
        for n in range(3):
            for i, v in enumerate(hex_decode(words[r, n])):
                assert q[8 * r + i, n] == v


def test_random_words_against_hex_reading():
    rng = np.random.default_rng(11)
    words = rng.integers(0, 2 ** 32, size=(64, 32), dtype=np.uint32)
    q = unpack_int4(words)
    for r in range(64):
        for n in range(32):
            assert q[8 * r:8 * r + 8, n].tolist() == hex_decode(words[r, n])


def test_round_trips():
    rng = np.random.default_rng(12)
    words = rng.integers(0, 2 ** 32, size=(1024, 1024), dtype=np.uint32)
    edge = np.array([[0, 0xFFFFFFFF, 0x80000000, 0x7FFFFFFF, 0x88888888, 0x77777777]], dtype=np.uint32)
    for w in (words, edge):
        assert np.array_equal(pack_int4(unpack_int4(w)), w)
    q = rng.integers(-8, 8, size=(256, 64))
    assert np.array_equal(unpack_int4(pack_int4(q)), q)
    assert unpack_int4(words).min() == -8 and unpack_int4(words).max() == 7


def test_pack_rejects_out_of_range():
    with pytest.raises(ValueError):
        pack_int4(np.full((8, 1), 8))
    with pytest.raises(ValueError):
        pack_int4(np.full((8, 1), -9))
    with pytest.raises(ValueError):
        pack_int4(np.zeros((7, 1), dtype=np.int64))
