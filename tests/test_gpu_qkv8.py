"""W8A16 fused QKV (kaio_qkv_w8a16) on the GPU against the CPU oracle (through the C ABI).

Same tolerance as W4A16, per output element: |y - Y*| <= ulp16(Y*) + 1e-5 * sum_k |x*w|,
against the unrounded float64 oracle value Y* (oracle.qkv.qkv_project with bits=8).
Cases whose exact result is representable in f16 are compared bit for bit.
"""
import numpy as np
import pytest
import torch

import int4_group_quantized_w4a16_amd as kaio
from int4_group_quantized_w4a16_amd import workloads
from oracle import compare
from oracle.int8 import pack_int8
from oracle.qkv import qkv_project
from tests.conftest import load_golden
from tests.gpu_util import DEV, NO_INT8_FORMS, TILE_FORMS, form_of, qkv_on_gpu, shape_for_form, to_dev, to_host
from tests.test_oracle_qkv8 import golden_inputs

pytestmark = pytest.mark.gpu


def run(x, w, s):
    return qkv_on_gpu(x, w, s, bits=8)


def check(outs, inp):
    ys, ts = qkv_project(inp.x, inp.w, inp.s, bits=8)
    worst = 0.0
    for name, o, y, t in zip("qkv", outs, ys, ts):
        bad, ratio = compare.excess(o, y, compare.qkv_tolerance(y, t))
        assert bad == 0, f"{name}: {bad} of {o.size} outside tolerance, max |d|/tol = {ratio:.3f}"
        worst = max(worst, ratio)
    return worst


def test_golden_handworked_bitwise():
    for case in load_golden("qkv8_handworked.json")["cases"]:
        x, w, s = golden_inputs(case)
        M, K = x.shape
        # pad 0: split-K kernel, one row tile; 20: two row tiles; 80: the tile kernel with one
        # output per workgroup (64 < m <= 128); 140: with all three (m > 128)
        for pad in (0, 20, 80, 140):
            xx = np.concatenate([x, np.zeros((pad, K), np.float16)]) if pad else x
            outs = run(xx, w, s)
            for p, o in zip("qkv", outs):
                want = np.array(case["expected"][p], dtype=np.float16)
                assert np.array_equal(o[:M].view(np.uint16), want.view(np.uint16)), (case["name"], p, pad)


@pytest.mark.parametrize("cfg", ["QKV8_TINY", "QKV8_DECODE", "QKV8_PREFILL"])
def test_workloads_all_outputs(cfg):
    c = getattr(workloads, cfg)
    inp = workloads.qkv8_inputs(c["M"], c["N"], c["K"], c["seed"])
    worst = check(run(inp.x, inp.w, inp.s), inp)
    print(f"{cfg} {c['M']}x{c['N']}x{c['K']} (all outputs): max |d|/tol = {worst:.3f}")


@pytest.mark.parametrize("M,N,K", [
    # split-K, m <= 8 (8 waves, several groups per wave), full and ragged strips
    (1, 100, 128), (7, 100, 256), (8, 64, 128), (8, 65, 384), (5, 72, 8320), (8, 64, 6272), (6, 65, 4096),
    # m <= 16, <= 32, <= 64, <= 128 (one, two and four row blocks), full and ragged
    (9, 100, 128), (16, 128, 512), (12, 64, 6272), (24, 200, 384), (32, 130, 384), (33, 64, 512),
    (48, 96, 1152), (64, 200, 256), (65, 64, 256), (100, 136, 384), (128, 64, 640), (40, 72, 4480),
    # tile kernel (test_every_tile_form covers each form), n % 8 == 0 and not, more than 32
    # groups (scale chunk reloads), groups split over two sets of waves (even counts) or not
    (129, 64, 256), (130, 200, 256), (300, 24, 640), (200, 1000, 1024), (129, 136, 8320),
    (1100, 1000, 4480), (1100, 1001, 256), (2100, 1000, 256), (2100, 1001, 128),
    (150, 264, 8448), (150, 261, 8448), (256, 4096, 4096),
])
def test_ragged_shapes(M, N, K):
    inp = workloads.qkv8_inputs(M, N, K, seed=M * 7919 + N * 31 + K + 1)
    check(run(inp.x, inp.w, inp.s), inp)


@pytest.mark.parametrize("aligned", [True, False], ids=["n%8==0", "n%8!=0"])
@pytest.mark.parametrize("form", [f for f in TILE_FORMS if f not in NO_INT8_FORMS],
                         ids=lambda f: f"{f[0]}w-{f[1]}rows-{f[2]}sets-{f[3]}outs")
def test_every_tile_form(form, aligned):
    # as for W4A16; INT8 lacks the forms whose rings would not fit in LDS
    shape = shape_for_form(form, 8, aligned)
    assert shape is not None, f"no problem selects {form}"
    M, N, K = shape
    assert form_of(kaio.kaio_qkv_plan(M, N, K, 8)) == form
    inp = workloads.qkv8_inputs(M, N, K, M * 7 + N * 3 + K + form[1] + form[3] + 1)
    worst = check(run(inp.x, inp.w, inp.s), inp)
    print(f"W8A16 {form} {M}x{N}x{K}: max |d|/tol = {worst:.3f}")


@pytest.mark.parametrize("M,N,K", [(512, 4096, 4096), (1024, 4096, 1024)])
def test_tile_kernel_super_block_grids_all_outputs(M, N, K):
    inp = workloads.qkv8_inputs(M, N, K, seed=M + N + K + 1)
    worst = check(run(inp.x, inp.w, inp.s), inp)
    print(f"W8A16 {M}x{N}x{K} (all outputs): max |d|/tol = {worst:.3f}")


@pytest.mark.parametrize("M", [4, 20, 160])
def test_identity_weights_reproduce_x(M):
    K = N = 512
    x = np.random.default_rng(M).standard_normal((M, K)).astype(np.float16)
    eye = np.eye(K, dtype=np.int64)
    ones = np.ones((K // 128, N), dtype=np.float16)
    q, k, v = run(x, [pack_int8(eye), pack_int8(-128 * eye), pack_int8(127 * eye)], [ones] * 3)
    x64 = x.astype(np.float64)
    assert np.array_equal(q.view(np.uint16), x.view(np.uint16))
    with np.errstate(over="ignore"):
        assert np.array_equal(k.view(np.uint16), (-128 * x64).astype(np.float16).view(np.uint16))
        assert np.array_equal(v.view(np.uint16), (127 * x64).astype(np.float16).view(np.uint16))


def test_one_hot_rows_read_back_every_weight():
    K, N = 256, 24
    inp = workloads.qkv8_inputs(1, N, K, 78)
    x = np.eye(K, dtype=np.float16)
    outs = run(x, inp.w, inp.s)
    ys, _ = qkv_project(x, inp.w, inp.s, bits=8)
    for o, y in zip(outs, ys):
        assert np.array_equal(o.view(np.uint16), y.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("M", [8, 40, 200])
def test_every_int8_value_and_extreme_scales_exact(M):
    # one x entry per row, a signed power of two, so that each output is the single product
    # x * q * s (<= 19 significant bits: exact in f32 on the GPU); its one rounding to f16
    # (RNE, subnormals and overflow included) must match the oracle bit for bit.  All 256
    # INT8 values meet scales at the f16 extremes.  M = 8, 40, 200: split-K with one and two
    # row tiles per wave, and the tile kernel.
    K, N = 256, 64
    kk, nn = np.meshgrid(np.arange(K), np.arange(N), indexing="ij")
    q = ((kk + 37 * nn) % 256) - 128
    w = pack_int8(q)
    svals = np.array([65504.0, 2.0 ** -14, 2.0 ** -24, 1.0, 0.00125, 3.0, 2.0 ** -20, 0.75])
    gg, nn2 = np.meshgrid(np.arange(K // 128), np.arange(N), indexing="ij")
    s = svals[(gg + nn2) % svals.size].astype(np.float16)
    x = np.zeros((M, K), dtype=np.float16)
    for i in range(M):
        x[i, (37 * i) % K] = (-1.0) ** i * 2.0 ** ((i % 15) - 10)
    outs = run(x, [w, w, w], [s, s, s])
    ys, _ = qkv_project(x, [w, w, w], [s, s, s], bits=8)
    for o, y in zip(outs, ys):
        with np.errstate(over="ignore"):
            want = y.astype(np.float16)
        assert np.array_equal(o.view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("M", [8, 64, 300])
def test_symmetry_swap_and_linearity(M):
    inp = workloads.qkv8_inputs(M, 192, 512, 98)
    q, k, v = run(inp.x, inp.w, inp.s)
    q2, k2, v2 = run(inp.x, [inp.w[1], inp.w[0], inp.w[2]], [inp.s[1], inp.s[0], inp.s[2]])
    assert np.array_equal(q2.view(np.uint16), k.view(np.uint16))
    assert np.array_equal(k2.view(np.uint16), q.view(np.uint16))
    e = run(inp.x, [inp.w[2]] * 3, [inp.s[2]] * 3)
    assert all(np.array_equal(a.view(np.uint16), v.view(np.uint16)) for a in e)
    d = run(inp.x, inp.w, [(2 * s.astype(np.float32)).astype(np.float16) for s in inp.s])
    for a, b in zip(d, (q, k, v)):
        normal = np.abs(b.astype(np.float64)) >= 2.0 ** -13
        assert np.array_equal(a[normal].astype(np.float64), 2 * b[normal].astype(np.float64))


def test_matches_int4_path_on_int4_range_weights():
    # INT4 values re-packed as INT8 (same q, same scales) must give the same outputs as the
    # W4A16 entry point where both run the same kernel configuration (m = 40: split-K with two
    # row tiles and two row blocks; m = 300: the tile kernel): the same exact products q * 2^-9
    # * x meet the MFMAs in the same k positions and are reduced in the same order, so the
    # results agree bit for bit.  (At m <= 16 the two split K over different wave counts.)
    from oracle.int4 import unpack_int4
    for M in (40, 300):
        inp4 = workloads.qkv_inputs(M, 256, 512, 12 + M)
        w8 = [pack_int8(unpack_int4(w).astype(np.int64)) for w in inp4.w]
        o4 = qkv_on_gpu(inp4.x, inp4.w, inp4.s, bits=4)
        o8 = run(inp4.x, w8, inp4.s)
        for a, b in zip(o4, o8):
            assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), M


def test_determinism_guard_bands_and_inputs_untouched():
    M, N, K = 72, 136, 384
    inp = workloads.qkv8_inputs(M, N, K, 6)
    x, w, s = to_dev(inp.x), [to_dev(a) for a in inp.w], [to_dev(a) for a in inp.s]
    copies = [t.clone() for t in [x, *w, *s]]
    pad = 4096
    results = []
    for _ in range(2):
        bufs = [torch.full((M * N + 2 * pad,), float("nan"), dtype=torch.float16, device=DEV) for _ in range(3)]
        outs = [b[pad:pad + M * N].view(M, N) for b in bufs]
        st = kaio.lib().kaio_qkv_w8a16(x.data_ptr(), *[t.data_ptr() for t in w], *[t.data_ptr() for t in s],
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


def test_errors_and_empty_reduction():
    x = torch.zeros((4, 256), dtype=torch.float16, device=DEV)
    w = torch.zeros((64, 16), dtype=torch.int32, device=DEV)
    s = torch.zeros((2, 16), dtype=torch.float16, device=DEV)
    o = [torch.zeros((4, 16), dtype=torch.float16, device=DEV) for _ in range(3)]
    L = kaio.lib()
    args = [x.data_ptr(), w.data_ptr(), w.data_ptr(), w.data_ptr(), s.data_ptr(), s.data_ptr(), s.data_ptr(),
            *[t.data_ptr() for t in o]]
    assert L.kaio_qkv_w8a16(*args, 4, 16, 256, 64, None) == 3
    assert L.kaio_qkv_w8a16(*args, 4, 16, 200, 128, None) == 2
    with pytest.raises(ValueError, match="rows, expected K/4"):
        kaio.kaio_qkv_w8a16(x, w[:32], w, w, s, s, s)
    outs = [torch.full((3, 40), float("nan"), dtype=torch.float16, device=DEV) for _ in range(3)]
    xe = torch.empty((3, 0), dtype=torch.float16, device=DEV)
    we = torch.empty((0, 40), dtype=torch.int32, device=DEV)
    se = torch.empty((0, 40), dtype=torch.float16, device=DEV)
    kaio.kaio_qkv_w8a16(xe, we, we, we, se, se, se, *outs)
    torch.cuda.synchronize()
    assert all((t == 0).all() for t in outs)
