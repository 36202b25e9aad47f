"""Pins for the W8A16 QKV oracle (oracle/qkv.py with bits=8).

* hand-worked cases (tests/golden/qkv8_handworked.json), exact;
* exact integer brute force with an independent (hex-digit) byte reader,
  summed in Python integers;
* one-hot rows of x read every weight back through the definition;
* identity weights (q = I, -128 I, 127 I) reproduce x exactly;
* linearity, symmetry, column locality; the K % 128 rule; the packed-row count.
"""
import numpy as np
import pytest

from int4_group_quantized_w4a16_amd.workloads import qkv8_inputs
from oracle.int8 import pack_int8
from oracle.qkv import qkv_project
from tests.conftest import load_golden

P = ("q", "k", "v")


def hex_q8(words):
    """int64 q[K, N] from packed words, read two hex digits per byte."""
    R, N = words.shape
    q = np.empty((4 * R, N), dtype=np.int64)
    for r in range(R):
        for n in range(N):
            d = format(int(words[r, n]), "08x")
            for i in range(4):
                v = int(d[6 - 2 * i:8 - 2 * i], 16)
                q[4 * r + i, n] = v - 256 if v >= 128 else v
    return q


def build_x8(rule, M, K):
    k = np.arange(K)
    if rule == "ones":
        return np.ones((M, K), dtype=np.float16)
    if rule == "row0: 1 where k%4==0, row1: 1 where k%4==3":
        return np.stack([(k % 4 == 0), (k % 4 == 3)]).astype(np.float16)
    raise KeyError(rule)


def golden_inputs(case):
    M, K, N = case["M"], case["K"], case["N"]
    x = build_x8(case["x_rule"], M, K)
    w, s = [], []
    for p in P:
        if "words" in case:
            row = np.array([int(h, 16) for h in case["words"][p]], dtype=np.uint32)
            w.append(np.tile(row, (K // 4, 1)))
        else:   # 32 packed rows per group of 128
            rows = [np.array([int(h, 16) for h in g], dtype=np.uint32) for g in case["per_group_words"][p]]
            w.append(np.concatenate([np.tile(r, (32, 1)) for r in rows]))
        s.append(np.array(case["scales"][p], dtype=np.float16))
    return x, w, s


def test_golden_handworked():
    for case in load_golden("qkv8_handworked.json")["cases"]:
        x, w, s = golden_inputs(case)
        ys, _ = qkv_project(x, w, s, bits=8)
        for p, y in zip(P, ys):
            assert np.array_equal(y, np.array(case["expected"][p])), (case["name"], p, y)


@pytest.mark.parametrize("M,N,K,seed", [(1, 1, 128, 1), (5, 3, 256, 2), (17, 33, 256, 3), (64, 48, 128, 4)])
def test_exact_integer_brute_force(M, N, K, seed):
    inp = qkv8_inputs(M, N, K, seed)
    ys, ts = qkv_project(inp.x, inp.w, inp.s, bits=8)
    # every f16 value is an integer multiple of 2**-24; sums in Python integers are exact
    xi = [[int(v) for v in row] for row in (inp.x.astype(np.float64) * 2.0 ** 24).astype(np.int64)]
    for p in range(3):
        q = hex_q8(inp.w[p])
        si = (inp.s[p].astype(np.float64) * 2.0 ** 24).astype(np.int64)
        wi = [[int(q[k, n]) * int(si[k // 128, n]) for n in range(N)] for k in range(K)]
        for m in range(M):
            for n in range(N):
                exact = sum(xi[m][k] * wi[k][n] for k in range(K))
                exact_abs = sum(abs(xi[m][k] * wi[k][n]) for k in range(K))
                t = exact_abs * 2.0 ** -48
                assert abs(ys[p][m, n] - exact * 2.0 ** -48) <= 1e-12 * t + 1e-300
                assert abs(ts[p][m, n] - t) <= 1e-12 * t + 1e-300


def test_one_hot_rows_read_back_every_weight():
    K, N = 256, 8
    inp = qkv8_inputs(1, N, K, 22)
    x = np.eye(K, dtype=np.float16)
    ys, _ = qkv_project(x, inp.w, inp.s, bits=8)
    for p in range(3):
        q = hex_q8(inp.w[p]).astype(np.float64)
        expect = q * inp.s[p].astype(np.float64)[np.arange(K) // 128]
        assert np.array_equal(ys[p], expect)
    # k = 203 sits in packed row 50, byte 3, group 1
    assert ys[1][203, 5] == hex_q8(inp.w[1][50:51, 5:6])[3, 0] * float(inp.s[1][1, 5])


def test_identity_weights_reproduce_x():
    rng = np.random.default_rng(6)
    K = N = 512
    x = rng.standard_normal((4, K)).astype(np.float16)
    eye = np.eye(K, dtype=np.int64)
    ones = np.ones((K // 128, N), dtype=np.float16)
    ys, _ = qkv_project(x, [pack_int8(eye), pack_int8(-128 * eye), pack_int8(127 * eye)], [ones] * 3, bits=8)
    assert np.array_equal(ys[0], x.astype(np.float64))
    assert np.array_equal(ys[1], -128 * x.astype(np.float64))
    assert np.array_equal(ys[2], 127 * x.astype(np.float64))


def test_linearity_symmetry_locality():
    inp = qkv8_inputs(6, 40, 384, 32)
    ys, ts = qkv_project(inp.x, inp.w, inp.s, bits=8)
    ys2, _ = qkv_project(inp.x, inp.w, [2 * s for s in inp.s], bits=8)
    ys3, _ = qkv_project((2 * inp.x.astype(np.float32)).astype(np.float16), inp.w, inp.s, bits=8)
    for p in range(3):
        assert np.array_equal(ys2[p], 2 * ys[p])
        assert np.array_equal(ys3[p], 2 * ys[p])
        assert np.all(np.abs(ys[p]) <= ts[p])
    ysw, _ = qkv_project(inp.x, [inp.w[1], inp.w[0], inp.w[2]], [inp.s[1], inp.s[0], inp.s[2]], bits=8)
    assert np.array_equal(ysw[0], ys[1]) and np.array_equal(ysw[1], ys[0]) and np.array_equal(ysw[2], ys[2])
    w0 = inp.w[0].copy()
    w0[:, 17] ^= np.uint32(0x5A5A5A5A)
    ysc, _ = qkv_project(inp.x, [w0, inp.w[1], inp.w[2]], inp.s, bits=8)
    keep = np.arange(40) != 17
    assert np.array_equal(ysc[0][:, keep], ys[0][:, keep])
    assert not np.array_equal(ysc[0][:, 17], ys[0][:, 17])


def test_shapes_k_rule_and_empty_k():
    # packed rows are K/4, not K/8
    inp = qkv8_inputs(2, 4, 256, 3)
    assert inp.w[0].shape == (64, 4)
    with pytest.raises(ValueError):
        qkv_project(inp.x, [w[:32] for w in inp.w], inp.s, bits=8)
    with pytest.raises(ValueError):
        qkv_project(inp.x, inp.w, inp.s, bits=4)
    for K in (64, 200):
        x = np.zeros((2, K), dtype=np.float16)
        w = [np.zeros((K // 4, 4), dtype=np.uint32)] * 3
        s = [np.zeros((max(K // 128, 1), 4), dtype=np.float16)] * 3
        with pytest.raises(ValueError):
            qkv_project(x, w, s, bits=8)
    ys, _ = qkv_project(np.zeros((3, 0), np.float16), [np.zeros((0, 5), np.uint32)] * 3,
                        [np.zeros((0, 5), np.float16)] * 3, bits=8)
    for y in ys:
        assert y.shape == (3, 5) and not y.any()
