"""Pins for the oracle's INT8 decoding (oracle/int8.py).

The convention (signed, low byte first, k = 4r + i) is read off hex digits
here -- byte i is the pair of hex digits 2i, 2i+1 counted from the right of the
word's 8-digit hex string -- a route that shares nothing with the oracle's
shift-and-mask decoder.
"""
import numpy as np
import pytest

from oracle.int8 import pack_int8, unpack_int8
from tests.conftest import load_golden


def hex_decode8(word):
    digits = format(int(word), "08x")
    vals = [int(digits[6 - 2 * i:8 - 2 * i], 16) for i in range(4)]
    return [v - 256 if v >= 128 else v for v in vals]


def test_golden_words():
    for case in load_golden("int8_words.json")["cases"]:
        word = int(case["word"], 16)
        q = np.array(case["q"], dtype=np.int64).reshape(4, 1)
        assert int(pack_int8(q)[0, 0]) == word, case
        assert unpack_int8(np.array([[word]], dtype=np.uint32))[:, 0].tolist() == case["q"]
        assert hex_decode8(word) == case["q"]


def test_every_byte_position_and_value():
    # 4 positions x 256 values, words built from hex strings (no shifts)
    for i in range(4):
        for v in range(256):
            digits = ["00"] * 4
            digits[3 - i] = format(v, "02x")
            word = int("".join(digits), 16)
            q = unpack_int8(np.array([[word]], dtype=np.uint32))[:, 0]
            expect = np.zeros(4, dtype=np.int64)
            expect[i] = v - 256 if v >= 128 else v
            assert q.tolist() == expect.tolist(), (i, v)


def test_layout_rows_and_columns():
    rng = np.random.default_rng(8)
    words = rng.integers(0, 2 ** 32, size=(5, 3), dtype=np.uint32)
    q = unpack_int8(words)
    assert q.shape == (20, 3)
    for r in range(5):
        for n in range(3):
            for i, v in enumerate(hex_decode8(words[r, n])):
                assert q[4 * r + i, n] == v


def test_random_words_against_hex_reading():
    rng = np.random.default_rng(13)
    words = rng.integers(0, 2 ** 32, size=(64, 32), dtype=np.uint32)
    q = unpack_int8(words)
    for r in range(64):
        for n in range(32):
            assert q[4 * r:4 * r + 4, n].tolist() == hex_decode8(words[r, n])


def test_round_trips():
    rng = np.random.default_rng(14)
    words = rng.integers(0, 2 ** 32, size=(1024, 1024), dtype=np.uint32)
    edge = np.array([[0, 0xFFFFFFFF, 0x80000000, 0x7FFFFFFF, 0x80808080, 0x7F7F7F7F]], dtype=np.uint32)
    for w in (words, edge):
        assert np.array_equal(pack_int8(unpack_int8(w)), w)
    q = rng.integers(-128, 128, size=(256, 64))
    assert np.array_equal(unpack_int8(pack_int8(q)), q)
    assert unpack_int8(words).min() == -128 and unpack_int8(words).max() == 127


def test_pack_rejects_out_of_range():
    with pytest.raises(ValueError):
        pack_int8(np.full((4, 1), 128))
    with pytest.raises(ValueError):
        pack_int8(np.full((4, 1), -129))
    with pytest.raises(ValueError):
        pack_int8(np.zeros((6, 1), dtype=np.int64))
