"""Pins for the QKV oracle (oracle/qkv.py).

* hand-worked cases (tests/golden/qkv_handworked.json), exact;
* exact integer brute force with an independent (hex-digit) nibble reader;
* one-hot rows of x read every weight back through the definition;
* identity weights reproduce x; linearity, symmetry and column locality;
* the K % 128 rule and the empty reduction.
"""
import numpy as np
import pytest

from oracle.int4 import pack_int4
from oracle.qkv import qkv_project
from tests.conftest import load_golden

P = ("q", "k", "v")


def hex_q(words):
    """int64 q[K, N] from packed words, read digit by digit from hex strings."""
    R, N = words.shape
    q = np.empty((8 * R, N), dtype=np.int64)
    for r in range(R):
        for n in range(N):
            d = format(int(words[r, n]), "08x")
            for i in range(8):
                v = int(d[7 - i], 16)
                q[8 * r + i, n] = v - 16 if v >= 8 else v
    return q


def build_x(rule, M, K):
    k = np.arange(K)
    if rule == "ones":
        return np.ones((M, K), dtype=np.float16)
    if rule == "row0 ones, row1 -0.5":
        return np.stack([np.ones(K), np.full(K, -0.5)]).astype(np.float16)
    if rule.startswith("row0: 1 where k%8==3"):
        return np.stack([(k % 8 == 3), (k % 8 == 7)]).astype(np.float16)
    if rule == "ones on k < 128, 0.5 on k >= 128":
        return np.where(k < 128, 1.0, 0.5).reshape(1, K).astype(np.float16)
    raise KeyError(rule)


def test_golden_handworked():
    for case in load_golden("qkv_handworked.json")["cases"]:
        M, K, N = case["M"], case["K"], case["N"]
        x = build_x(case["x_rule"], M, K)
        w, s = [], []
        for p in P:
            if "words" in case:
                row = np.array([int(h, 16) for h in case["words"][p]], dtype=np.uint32)
                w.append(np.tile(row, (K // 8, 1)))
            else:
                rows = [np.array([int(h, 16) for h in g], dtype=np.uint32) for g in case["per_group_words"][p]]
                w.append(np.concatenate([np.tile(r, (16, 1)) for r in rows]))
            s.append(np.array(case["scales"][p], dtype=np.float16))
        ys, _ = qkv_project(x, w, s)
        for p, y in zip(P, ys):
            assert np.array_equal(y, np.array(case["expected"][p])), (case["name"], p, y)


@pytest.mark.parametrize("M,N,K,seed", [(1, 1, 128, 1), (5, 3, 256, 2), (17, 33, 256, 3), (128, 128, 128, 4)])
def test_exact_integer_brute_force(M, N, K, seed):
    from int4_group_quantized_w4a16_amd.workloads import qkv_inputs
    inp = qkv_inputs(M, N, K, seed)
    ys, ts = qkv_project(inp.x, inp.w, inp.s)
    # every f16 value is an integer multiple of 2**-24, exactly
    xi = (inp.x.astype(np.float64) * 2.0 ** 24).astype(np.int64)
    for p in range(3):
        q = hex_q(inp.w[p])
        si = (inp.s[p].astype(np.float64) * 2.0 ** 24).astype(np.int64)
        wi = q * si[np.arange(K) // 128]              # integer multiples of 2**-24
        exact = xi @ wi                                # integer multiples of 2**-48, exact in int64 here
        exact_abs = np.abs(xi) @ np.abs(wi)
        y_exact = exact.astype(np.float64) * 2.0 ** -48
        t_exact = exact_abs.astype(np.float64) * 2.0 ** -48
        assert np.all(np.abs(ys[p] - y_exact) <= 1e-12 * t_exact + 1e-300)
        assert np.all(np.abs(ts[p] - t_exact) <= 1e-12 * t_exact + 1e-300)


def test_one_hot_rows_read_back_every_weight():
    from int4_group_quantized_w4a16_amd.workloads import qkv_inputs
    K, N = 256, 8
    inp = qkv_inputs(1, N, K, 21)
    x = np.eye(K, dtype=np.float16)                   # row k is e_k
    ys, _ = qkv_project(x, inp.w, inp.s)
    for p in range(3):
        q = hex_q(inp.w[p]).astype(np.float64)
        expect = q * inp.s[p].astype(np.float64)[np.arange(K) // 128]
        assert np.array_equal(ys[p], expect)
    # k = 200 sits in packed row 25, nibble 0, group 1
    assert ys[0][200, 3] == hex_q(inp.w[0][25:26, 3:4])[0, 0] * float(inp.s[0][1, 3])


def test_identity_weights_reproduce_x():
    rng = np.random.default_rng(5)
    K = N = 512
    x = rng.standard_normal((4, K)).astype(np.float16)
    eye = np.eye(K, dtype=np.int64)
    ones = np.ones((K // 128, N), dtype=np.float16)
    ys, _ = qkv_project(x, [pack_int4(eye), pack_int4(-eye), pack_int4(7 * eye)], [ones] * 3)
    assert np.array_equal(ys[0], x.astype(np.float64))
    assert np.array_equal(ys[1], -x.astype(np.float64))
    assert np.array_equal(ys[2], 7 * x.astype(np.float64))


def test_linearity_symmetry_locality():
    from int4_group_quantized_w4a16_amd.workloads import qkv_inputs
    inp = qkv_inputs(6, 40, 384, 31)
    ys, ts = qkv_project(inp.x, inp.w, inp.s)
    ys2, _ = qkv_project(inp.x, inp.w, [2 * s for s in inp.s])
    ys3, _ = qkv_project((2 * inp.x.astype(np.float32)).astype(np.float16), inp.w, inp.s)
    for p in range(3):
        assert np.array_equal(ys2[p], 2 * ys[p])
        assert np.array_equal(ys3[p], 2 * ys[p])
        assert np.all(np.abs(ys[p]) <= ts[p])
    # swapping the (weight, scale) pairs of two projections swaps their outputs
    ysw, _ = qkv_project(inp.x, [inp.w[1], inp.w[0], inp.w[2]], [inp.s[1], inp.s[0], inp.s[2]])
    assert np.array_equal(ysw[0], ys[1]) and np.array_equal(ysw[1], ys[0]) and np.array_equal(ysw[2], ys[2])
    # equal weights and scales give equal outputs
    yse, _ = qkv_project(inp.x, [inp.w[0]] * 3, [inp.s[0]] * 3)
    assert np.array_equal(yse[0], yse[1]) and np.array_equal(yse[1], yse[2])
    # changing one column changes only that column
    w0 = inp.w[0].copy()
    w0[:, 17] ^= np.uint32(0x5A5A5A5A)
    ysc, _ = qkv_project(inp.x, [w0, inp.w[1], inp.w[2]], inp.s)
    keep = np.arange(40) != 17
    assert np.array_equal(ysc[0][:, keep], ys[0][:, keep])
    assert not np.array_equal(ysc[0][:, 17], ys[0][:, 17])


def test_k_multiple_of_128_and_empty_k():
    for K in (64, 200):
        x = np.zeros((2, K), dtype=np.float16)
        w = [np.zeros((K // 8, 4), dtype=np.uint32)] * 3
        s = [np.zeros((max(K // 128, 1), 4), dtype=np.float16)] * 3
        with pytest.raises(ValueError):
            qkv_project(x, w, s)
    ys, _ = qkv_project(np.zeros((3, 0), np.float16), [np.zeros((0, 5), np.uint32)] * 3,
                        [np.zeros((0, 5), np.float16)] * 3)
    for y in ys:
        assert y.shape == (3, 5) and not y.any()


def test_row_subset_matches_full():
    from int4_group_quantized_w4a16_amd.workloads import qkv_inputs
    inp = qkv_inputs(20, 24, 256, 41)
    ys, ts = qkv_project(inp.x, inp.w, inp.s)
    rows = np.array([19, 0, 7])
    ysr, tsr = qkv_project(inp.x, inp.w, inp.s, rows=rows)
    for p in range(3):
        assert np.array_equal(ysr[p], ys[p][rows]) and np.array_equal(tsr[p], ts[p][rows])
