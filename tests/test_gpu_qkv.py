"""W4A16 fused QKV on the GPU against the CPU oracle (through the C ABI).

Tolerance (per output element): |y - Y*| <= ulp16(Y*) + 1e-5 * sum_k |x*w|,
against the unrounded float64 oracle value Y*.  Cases whose exact result is
representable in f16 are compared bit for bit.
"""
import numpy as np
import pytest
import torch

import int4_group_quantized_w4a16_amd as kaio
from int4_group_quantized_w4a16_amd import workloads
from oracle import compare
from oracle.int4 import pack_int4, unpack_int4
from oracle.qkv import qkv_project
from tests.conftest import load_golden
from tests.gpu_util import DEV, TILE_FORMS, form_of, qkv_on_gpu, shape_for_form, to_dev, to_host
from tests.test_oracle_qkv import build_x

pytestmark = pytest.mark.gpu


def check(outs, inp, rows=None):
    ys, ts = qkv_project(inp.x, inp.w, inp.s, rows=rows)
    worst = 0.0
    for name, o, y, t in zip("qkv", outs, ys, ts):
        got = o if rows is None else o[rows]
        bad, ratio = compare.excess(got, y, compare.qkv_tolerance(y, t))
        assert bad == 0, f"{name}: {bad} of {got.size} outside tolerance, max |d|/tol = {ratio:.3f}"
        worst = max(worst, ratio)
    return worst


def test_golden_handworked_bitwise():
    for case in load_golden("qkv_handworked.json")["cases"]:
        M, K, N = case["M"], case["K"], case["N"]
        x = build_x(case["x_rule"], M, K)
        w, s = [], []
        for p in "qkv":
            if "words" in case:
                row = np.array([int(h, 16) for h in case["words"][p]], dtype=np.uint32)
                w.append(np.tile(row, (K // 8, 1)))
            else:
                rows = [np.array([int(h, 16) for h in g], dtype=np.uint32) for g in case["per_group_words"][p]]
                w.append(np.concatenate([np.tile(r, (16, 1)) for r in rows]))
            s.append(np.array(case["scales"][p], dtype=np.float16))
        # pad 20 runs the split-K kernel with two row tiles per wave, pad 80 the tile kernel with one
        # output per workgroup (64 < m <= 128), pad 140 the tile kernel with all three (m > 128)
        for pad in (0, 20, 80, 140):
            xx = np.concatenate([x, np.zeros((pad, K), np.float16)]) if pad else x
            outs = qkv_on_gpu(xx, w, s)
            for p, o in zip("qkv", outs):
                want = np.array(case["expected"][p], dtype=np.float16)
                assert np.array_equal(o[:M].view(np.uint16), want.view(np.uint16)), (case["name"], p, pad)


def test_tiny_config_all_outputs():
    inp = workloads.qkv_inputs(**{k: v for k, v in workloads.QKV_TINY.items()})
    worst = check(qkv_on_gpu(inp.x, inp.w, inp.s), inp)
    print(f"tiny 16x512x512: max |d|/tol = {worst:.3f}")


@pytest.mark.parametrize("M,N,K", [
    (1, 100, 128), (7, 100, 256), (8, 64, 128), (8, 65, 384), (9, 100, 128), (16, 8, 128),
    (17, 72, 384), (128, 64, 128), (129, 65, 128), (130, 200, 256), (1, 1, 128), (300, 24, 640),
    (64, 4, 128), (3, 4099, 256), (200, 1000, 1024),
    # more than 32 groups: the tile kernel reloads its per-chunk scales
    (33, 72, 4480), (129, 136, 8320), (20, 12, 4224),
    # split-K row-tile boundaries (1 and 2 row tiles, 1 and 2 row blocks), full and ragged strips,
    # then the tile kernel with one output per workgroup (four sets of 64-row tiles where k / 128
    # divides by 4, 96- and 128-row tiles), then with three
    (16, 128, 512), (17, 64, 256), (24, 200, 384), (32, 130, 384), (33, 64, 512), (48, 96, 1152),
    (63, 40, 256), (64, 200, 256), (65, 64, 256), (96, 136, 384), (127, 72, 256), (128, 64, 640),
    (129, 64, 256),
    # tile kernel on larger grids, ragged and n % 8 != 0, one or two groups (test_every_tile_form
    # covers each form of the tile kernel)
    (1100, 1000, 256), (1100, 1001, 128), (2100, 1000, 256), (2100, 1001, 128),
    # more than 32 groups (scale chunk reloads), per set where the groups are split over two sets
    # of waves (66 and 34 groups: 33 and 17 per set), and odd counts (97, 35: one set)
    (200, 520, 12416), (1100, 1000, 4480), (150, 264, 8448), (150, 261, 8448),
    (1100, 1000, 4352), (1100, 1001, 4352),
    # split-K with n % 64 != 0 but n % 4 == 0: whole-vector loads on every strip, the last strip's
    # lanes past n loading the last valid columns (decode width, and K > 4096)
    (8, 4088, 4096), (5, 1000, 4096), (16, 4040, 4608), (30, 1004, 512),
    # the same with trimmed loads past a wave's groups (m <= 16, k > 4096) and with every group of a
    # wave in flight (m <= 8, 40 to 64 groups)
    (8, 1004, 4480), (16, 1000, 4480), (5, 1000, 6144), (8, 4088, 8192), (1, 100, 7168),
    # n % 4 != 0: column-by-column loads, columns past n loading column n - 1
    (8, 4095, 4096), (13, 1001, 640), (40, 999, 384),
    # four sets of waves over 64-row tiles, one output per workgroup: ragged rows and columns,
    # n % 8 != 0, several groups per set
    (33, 72, 512), (47, 130, 1024), (64, 61, 2048), (50, 4096, 1536),
    # split-K: waves with exactly two groups on ragged strips (the straight-line path), and
    # waves with three or more groups, odd counts included (the loop; 8 and 16 x rows kept)
    (6, 65, 4096), (15, 100, 4096), (5, 72, 8320), (8, 64, 6272), (12, 64, 6272), (40, 72, 4480),
    # m <= 8 on whole strips with 40 to 64 groups: all of a wave's groups in flight, x through direct
    # LDS loads (40 and 41 groups: waves with 2 and 3; 48: 3 each; 49 above: 3 and 4; 64: 4 each);
    # 33 groups stays on the two-chunk path
    (8, 128, 5120), (3, 64, 5248), (7, 192, 6144), (1, 64, 8192), (8, 4096, 8192), (8, 128, 4224),
])
def test_ragged_shapes(M, N, K):
    inp = workloads.qkv_inputs(M, N, K, seed=M * 7919 + N * 31 + K)
    check(qkv_on_gpu(inp.x, inp.w, inp.s), inp)


def test_decode_config_all_outputs():
    c = workloads.QKV_DECODE
    inp = workloads.qkv_inputs(c["M"], c["N"], c["K"], c["seed"])
    worst = check(qkv_on_gpu(inp.x, inp.w, inp.s), inp)
    print(f"decode 8x4096x4096: max |d|/tol = {worst:.3f}")


def test_prefill_config_all_outputs():
    # every one of the 3 x 2048 x 4096 outputs of the prefill workload (tile kernel, 8 waves,
    # XCD super-block tile order: 16 row tiles x 32 column tiles)
    c = workloads.QKV_PREFILL
    inp = workloads.qkv_inputs(c["M"], c["N"], c["K"], c["seed"])
    outs = qkv_on_gpu(inp.x, inp.w, inp.s)
    worst = check(outs, inp)
    print(f"prefill 2048x4096x4096 (all outputs): max |d|/tol = {worst:.3f}")


@pytest.mark.parametrize("M,N,K", [
    (256, 4096, 4096),    # 64-row tiles (4 x 64 tiles of 64 x 64), groups split over two sets of 4 waves
    (200, 4096, 4096),    # the same with a ragged last row tile (8 of its 64 rows)
    (512, 4096, 4096),    # 4 x 64 tiles of 128 x 64 in 4 x 8 super-blocks, groups split over two sets
    (1024, 4096, 1024),   # 8-wave tile kernel: 8 x 32 tiles of 128 x 128, walked in 4 x 8 super-blocks
])
def test_tile_kernel_super_block_grids_all_outputs(M, N, K):
    assert form_of(kaio.kaio_qkv_plan(M, N, K)) == {256: (4, 64, 2, 3), 200: (4, 64, 2, 3), 512: (4, 128, 2, 3),
                                                    1024: (8, 128, 1, 3)}[M]
    inp = workloads.qkv_inputs(M, N, K, seed=M + N + K)
    worst = check(qkv_on_gpu(inp.x, inp.w, inp.s), inp)
    print(f"{M}x{N}x{K} (all outputs): max |d|/tol = {worst:.3f}")


@pytest.mark.parametrize("aligned", [True, False], ids=["n%8==0", "n%8!=0"])
@pytest.mark.parametrize("form", TILE_FORMS, ids=lambda f: f"{f[0]}w-{f[1]}rows-{f[2]}sets-{f[3]}outs")
def test_every_tile_form(form, aligned):
    # the smallest problem of a coarse grid that the plan runs in this form: m ragged against the
    # tile height, n ragged against the tile width
    shape = shape_for_form(form, 4, aligned)
    assert shape is not None, f"no problem selects {form}"
    M, N, K = shape
    assert form_of(kaio.kaio_qkv_plan(M, N, K)) == form
    inp = workloads.qkv_inputs(M, N, K, seed=M * 7 + N * 3 + K + form[1] + form[3])
    worst = check(qkv_on_gpu(inp.x, inp.w, inp.s), inp)
    print(f"{form} {M}x{N}x{K}: max |d|/tol = {worst:.3f}")


@pytest.mark.parametrize("M,N,K", [(8, 4088, 4096), (8, 4095, 4096), (16, 1000, 4480), (8, 4088, 8192),
                                   (5, 1004, 6144), (30, 996, 512)])
def test_ragged_columns_match_the_padded_problem(M, N, K):
    # split-K on a partial last strip (n % 64 != 0; whole-vector loads with the lanes past n
    # loading the last columns, or column-by-column loads for n % 4 != 0, on the two-chunk,
    # trimmed and all-groups forms): the columns below n are bit-identical to those of the same
    # problem padded to whole strips (MFMA columns do not mix and the reduction order does not
    # depend on n)
    Np = (N + 63) // 64 * 64
    full = workloads.qkv_inputs(M, Np, K, seed=M * 13 + N + K)
    ragged = qkv_on_gpu(full.x, [a[:, :N] for a in full.w], [a[:, :N] for a in full.s])
    padded = qkv_on_gpu(full.x, full.w, full.s)
    for r, p in zip(ragged, padded):
        assert np.array_equal(r.view(np.uint16), p[:, :N].view(np.uint16))


@pytest.mark.parametrize("M,N,K", [(2048, 4095, 1024), (100, 4092, 4096), (40, 4090, 4096), (300, 1001, 512)])
def test_tile_columns_match_the_padded_problem(M, N, K):
    # the tile kernel with n % 8 != 0 (4-byte weight loads, column-guarded scales and stores) in the
    # three-output, one-output and four-set forms: the columns below n are bit-identical to those
    # of the same problem padded to n % 128 == 0, which runs the same form with 16-byte loads
    Np = (N + 127) // 128 * 128
    assert form_of(kaio.kaio_qkv_plan(M, N, K)) == form_of(kaio.kaio_qkv_plan(M, Np, K))
    full = workloads.qkv_inputs(M, Np, K, seed=M * 17 + N + K)
    ragged = qkv_on_gpu(full.x, [a[:, :N] for a in full.w], [a[:, :N] for a in full.s])
    padded = qkv_on_gpu(full.x, full.w, full.s)
    for r, p in zip(ragged, padded):
        assert np.array_equal(r.view(np.uint16), p[:, :N].view(np.uint16))


@pytest.mark.parametrize("M", [8, 40, 200])
def test_non_finite_inputs_stay_in_their_rows(M):
    # IEEE propagation, row by row: a NaN in x row 1 makes that row NaN everywhere; +inf in row 2
    # at k0 gives +-inf by the sign of q[k0, n] (NaN where that weight is 0); every other row is
    # finite and within tolerance (MFMA rows do not mix).  M = 8, 40: split-K kernel; 200: tile.
    N, K, k0 = 72, 384, 137
    inp = workloads.qkv_inputs(M, N, K, seed=600 + M)
    x = inp.x.copy()
    x[1, 5] = np.float16(np.nan)
    x[2, k0] = np.float16(np.inf)
    outs = qkv_on_gpu(x, inp.w, inp.s)
    finite = [r for r in range(M) if r not in (1, 2)]
    ys, ts = qkv_project(inp.x[finite], inp.w, inp.s)
    for o, wq, y, t in zip(outs, inp.w, ys, ts):
        assert np.isnan(o[1]).all()
        q = unpack_int4(wq)[k0]                      # signed INT4 values of packed row k0 // 8
        assert np.array_equal(np.isnan(o[2]), q == 0)
        assert np.array_equal(np.sign(o[2][q != 0]), np.sign(q[q != 0]).astype(np.float16))
        assert np.isinf(o[2][q != 0]).all()
        bad, ratio = compare.excess(o[finite], y, compare.qkv_tolerance(y, t))
        assert bad == 0, f"{bad} finite outputs outside tolerance, max |d|/tol = {ratio:.3f}"


@pytest.mark.parametrize("M", [4, 40])
def test_identity_weights_reproduce_x(M):
    K = N = 512
    x = np.random.default_rng(M).standard_normal((M, K)).astype(np.float16)
    eye = np.eye(K, dtype=np.int64)
    ones = np.ones((K // 128, N), dtype=np.float16)
    q, k, v = qkv_on_gpu(x, [pack_int4(eye), pack_int4(-eye), pack_int4(7 * eye)], [ones] * 3)
    assert np.array_equal(q.view(np.uint16), x.view(np.uint16))
    assert np.array_equal(k.view(np.uint16), (-x).view(np.uint16))
    assert np.array_equal(v.view(np.uint16), (7 * x.astype(np.float64)).astype(np.float16).view(np.uint16))


def test_one_hot_rows_read_back_every_weight():
    K, N = 256, 24
    inp = workloads.qkv_inputs(1, N, K, 77)
    x = np.eye(K, dtype=np.float16)
    outs = qkv_on_gpu(x, inp.w, inp.s)
    ys, _ = qkv_project(x, inp.w, inp.s)
    for o, y in zip(outs, ys):
        assert np.array_equal(o.view(np.uint16), y.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("M", [8, 40, 200])
def test_every_int4_value_and_extreme_scales_exact(M):
    # one x entry per row, a signed power of two, so that each output is a single product
    # x * q * s with at most 15 significant bits: exact in f32 on the GPU, and the one
    # rounding to f16 (RNE, subnormals and overflow included) must match the oracle bit for bit.
    # Every q in [-8, 7] meets scales at the f16 extremes (largest normal, smallest normal,
    # smallest subnormal).  M = 8, 40 and 200 run the split-K kernel with one and with two row
    # tiles per wave and the tile kernel.
    K, N = 256, 64
    kk, nn = np.meshgrid(np.arange(K), np.arange(N), indexing="ij")
    q = ((kk + 3 * nn) % 16) - 8
    w = pack_int4(q)
    svals = np.array([65504.0, 2.0 ** -14, 2.0 ** -24, 1.0, 0.005, 3.0, 2.0 ** -20, 0.75])
    gg, nn2 = np.meshgrid(np.arange(K // 128), np.arange(N), indexing="ij")
    s = svals[(gg + nn2) % svals.size].astype(np.float16)
    x = np.zeros((M, K), dtype=np.float16)
    for i in range(M):
        x[i, (37 * i) % K] = (-1.0) ** i * 2.0 ** ((i % 15) - 10)
    outs = qkv_on_gpu(x, [w, w, w], [s, s, s])
    ys, _ = qkv_project(x, [w, w, w], [s, s, s])
    for o, y in zip(outs, ys):
        with np.errstate(over="ignore"):   # products beyond 65504 round to +-inf, as on the GPU
            want = y.astype(np.float16)
        assert np.array_equal(o.view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("M", [8, 64])
def test_symmetry_swap_and_linearity(M):
    inp = workloads.qkv_inputs(M, 192, 512, 99)
    q, k, v = qkv_on_gpu(inp.x, inp.w, inp.s)
    q2, k2, v2 = qkv_on_gpu(inp.x, [inp.w[1], inp.w[0], inp.w[2]], [inp.s[1], inp.s[0], inp.s[2]])
    assert np.array_equal(q2.view(np.uint16), k.view(np.uint16))
    assert np.array_equal(k2.view(np.uint16), q.view(np.uint16))
    e = qkv_on_gpu(inp.x, [inp.w[2]] * 3, [inp.s[2]] * 3)
    assert all(np.array_equal(a.view(np.uint16), v.view(np.uint16)) for a in e)
    d = qkv_on_gpu(inp.x, inp.w, [(2 * s.astype(np.float32)).astype(np.float16) for s in inp.s])
    for a, b in zip(d, (q, k, v)):
        normal = np.abs(b.astype(np.float64)) >= 2.0 ** -13
        assert np.array_equal(a[normal].astype(np.float64), 2 * b[normal].astype(np.float64))


def test_determinism_guard_bands_and_inputs_untouched():
    M, N, K = 72, 136, 384
    inp = workloads.qkv_inputs(M, N, K, 5)
    x, w, s = to_dev(inp.x), [to_dev(a) for a in inp.w], [to_dev(a) for a in inp.s]
    copies = [t.clone() for t in [x, *w, *s]]
    pad = 4096
    results = []
    for _ in range(2):
        bufs = [torch.full((M * N + 2 * pad,), float("nan"), dtype=torch.float16, device=DEV) for _ in range(3)]
        outs = [b[pad:pad + M * N].view(M, N) for b in bufs]
        # the binding insists on zero-offset tensors; call the C ABI directly
        st = kaio.lib().kaio_qkv_w4a16(x.data_ptr(), *[t.data_ptr() for t in w], *[t.data_ptr() for t in s],
                                       *[o.data_ptr() for o in outs], M, N, K, 128, None)
        assert st == 0, kaio.kaio_last_error()
        torch.cuda.synchronize()
        for b in bufs:
            assert torch.isnan(b[:pad]).all() and torch.isnan(b[pad + M * N:]).all()
        results.append([to_host(o) for o in outs])
    for a, b in zip(*results):
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    for t, c in zip([x, *w, *s], copies):
        assert torch.equal(t, c)
    check(results[0], inp)


@pytest.mark.parametrize("M", [3, 50])
def test_empty_reduction_writes_zeros(M):
    N = 40
    outs = [torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV) for _ in range(3)]
    x = torch.empty((M, 0), dtype=torch.float16, device=DEV)
    w = torch.empty((0, N), dtype=torch.int32, device=DEV)
    s = torch.empty((0, N), dtype=torch.float16, device=DEV)
    kaio.kaio_qkv_w4a16(x, w, w, w, s, s, s, *outs)
    torch.cuda.synchronize()
    for o in outs:
        assert (o == 0).all()


def test_errors_on_device():
    x = torch.zeros((4, 256), dtype=torch.float16, device=DEV)
    w = torch.zeros((32, 16), dtype=torch.int32, device=DEV)
    s = torch.zeros((2, 16), dtype=torch.float16, device=DEV)
    o = [torch.zeros((4, 16), dtype=torch.float16, device=DEV) for _ in range(3)]
    L = kaio.lib()
    args = [x.data_ptr(), w.data_ptr(), w.data_ptr(), w.data_ptr(), s.data_ptr(), s.data_ptr(), s.data_ptr(),
            *[t.data_ptr() for t in o]]
    assert L.kaio_qkv_w4a16(*args, 4, 16, 256, 64, None) == 3
    assert L.kaio_qkv_w4a16(*args, 4, 16, 200, 128, None) == 2
    assert L.kaio_qkv_w4a16(*args[:7], o[0].data_ptr(), o[0].data_ptr(), o[2].data_ptr(), 4, 16, 256, 128, None) == 1
    with pytest.raises(ValueError, match="rows, expected K/8"):
        kaio.kaio_qkv_w4a16(x, w[:16], w, w, s, s, s)
    with pytest.raises(ValueError, match="N mismatch"):
        kaio.kaio_qkv_w4a16(x, w, w, w[:, :8].contiguous(), s, s, s)


@pytest.mark.parametrize("M", [16, 32, 64, 96, 128])
def test_batched_decode_full_size(M):
    # the split-K kernel (m <= 32), the one-output tile kernel with four sets (m = 64) and with
    # 96 and 128 rows, at the decode width (N = K = 4096), every output checked
    N = K = 4096
    inp = workloads.qkv_inputs(M, N, K, seed=4000 + M)
    check(qkv_on_gpu(inp.x, inp.w, inp.s), inp)
