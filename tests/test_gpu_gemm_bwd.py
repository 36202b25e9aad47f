"""GEMM backward on the GPU against the CPU oracle (through the C ABI).

grad_a = f16(f16(G) . B^T), grad_b = f16(A^T . f16(G)); tolerance per element
|d - Y*| <= ulp16(Y*) + 1e-5 * T against the unrounded float64 oracle value.
Cases whose exact results are representable in f16 are compared bit for bit.
Shapes cover the direct-to-LDS paths (strides multiples of 8; whole 64-k stages and a
ragged last stage) and the register-staged MFMA kernel that takes any shape, for each gradient
(n or k not a multiple of 8), over one tile and over several.
"""
import numpy as np
import pytest
import torch

import int4_group_quantized_w4a16_amd as kaio
from int4_group_quantized_w4a16_amd import workloads
from oracle import compare
from oracle.gemm_bwd import gemm_bwd, gemm_bwd_at
from tests.conftest import hexfloat, load_golden
from tests.gpu_util import DEV, to_dev, to_host

pytestmark = pytest.mark.gpu


def run(a, b, g):
    ga, gb = kaio.kaio_gemm_f16f32_bwd(to_dev(a), to_dev(b), to_dev(g))
    torch.cuda.synchronize()
    return to_host(ga), to_host(gb)


def inputs(m, n, k, seed):
    a, b = workloads.gemm_inputs(m, n, k, seed)
    g = np.random.default_rng(seed + 1).standard_normal((m, n)).astype(np.float32)
    return a, b, g


def check(got, a, b, g):
    (da, ta), (db, tb) = gemm_bwd(a, b, g)
    for name, x, y, t in (("grad_a", got[0], da, ta), ("grad_b", got[1], db, tb)):
        bad, ratio = compare.excess(x, y, compare.f16_tolerance(y, t))
        assert bad == 0, f"{name}: {bad} of {x.size} outside tolerance, max ratio {ratio:.3f}"


def test_golden_handworked_bitwise():
    for case in load_golden("gemm_bwd_handworked.json")["cases"]:
        mat = lambda rows, dt: np.array([[hexfloat(v) for v in r] for r in rows], dtype=dt)
        ga, gb = run(mat(case["a"], np.float16), mat(case["b"], np.float16), mat(case["g"], np.float32))
        assert np.array_equal(ga, mat(case["da"], np.float16))
        assert np.array_equal(gb, mat(case["db"], np.float16))


@pytest.mark.parametrize("M,N,K", [
    (256, 256, 256),      # both gradients on the direct-to-LDS path
    (320, 192, 520),      # both direct, ragged output tiles
    (300, 128, 136),      # grad_a direct, grad_b direct with a ragged last stage (m % 64 != 0)
    (192, 72, 264),       # grad_a direct with a ragged last stage (n % 64 != 0), grad_b direct
    (1000, 520, 776), (37, 200, 64), (65, 72, 80), (2, 8, 8),   # both ragged
    (5, 7, 9), (1, 64, 1), (64, 64, 8), (130, 64, 3),           # n or k % 8 != 0: the register-staged kernel
    # the register-staged kernel over several 256 x 256 tiles and 64-k stages: both gradients
    # (n % 8 != 0), grad_b alone (k % 8 != 0), both with every extent odd
    (270, 1030, 512), (520, 600, 260), (300, 1001, 515),
])
def test_shapes(M, N, K):
    a, b, g = inputs(M, N, K, M * 31 + N * 7 + K)
    check(run(a, b, g), a, b, g)


def test_exact_integers_bitwise():
    # small integers: every sum is exact in f32 and f16, so results are bit-exact
    rng = np.random.default_rng(21)
    M, N, K = 128, 256, 72
    a = rng.integers(-4, 5, size=(M, K)).astype(np.float16)
    b = rng.integers(-4, 5, size=(K, N)).astype(np.float16)
    g = rng.integers(-4, 5, size=(M, N)).astype(np.float32)
    ga, gb = run(a, b, g)
    (da, _), (db, _) = gemm_bwd(a, b, g)
    assert np.array_equal(ga, da.astype(np.float16)) and np.array_equal(gb, db.astype(np.float16))


def test_ragged_exact_integers_bitwise():
    # both gradients through the ragged last stage (n = 72, m = 100): exact small-integer sums
    rng = np.random.default_rng(23)
    M, N, K = 100, 72, 200
    a = rng.integers(-4, 5, size=(M, K)).astype(np.float16)
    b = rng.integers(-4, 5, size=(K, N)).astype(np.float16)
    g = rng.integers(-4, 5, size=(M, N)).astype(np.float32)
    ga, gb = run(a, b, g)
    (da, _), (db, _) = gemm_bwd(a, b, g)
    assert np.array_equal(ga, da.astype(np.float16)) and np.array_equal(gb, db.astype(np.float16))


def test_any_shape_exact_integers_bitwise():
    # n and k odd: both gradients on the register-staged kernel, exact small-integer sums
    rng = np.random.default_rng(25)
    M, N, K = 100, 275, 333
    a = rng.integers(-4, 5, size=(M, K)).astype(np.float16)
    b = rng.integers(-4, 5, size=(K, N)).astype(np.float16)
    g = rng.integers(-4, 5, size=(M, N)).astype(np.float32)
    ga, gb = run(a, b, g)
    (da, _), (db, _) = gemm_bwd(a, b, g)
    assert np.array_equal(ga, da.astype(np.float16)) and np.array_equal(gb, db.astype(np.float16))


def test_large_odd_sampled():
    # every extent odd at a large size (4 x 8 and 5 x 8 output tiles, 16-33 stages)
    M, N, K = 1025, 2047, 1279
    a, b, g = inputs(M, N, K, 4244)
    ga, gb = run(a, b, g)
    rng = np.random.default_rng(4245)
    ra, ca = rng.integers(0, M, 2048), rng.integers(0, K, 2048)
    rb, cb = rng.integers(0, K, 2048), rng.integers(0, N, 2048)
    (pa, ta), (pb, tb) = gemm_bwd_at(a, b, g, ra, ca, rb, cb)
    for name, x, y, t in (("grad_a", ga[ra, ca], pa, ta), ("grad_b", gb[rb, cb], pb, tb)):
        bad, ratio = compare.excess(x, y, compare.f16_tolerance(y, t))
        assert bad == 0, f"{name}: {bad} outside tolerance, max ratio {ratio:.3f}"


def test_large_ragged_sampled():
    # m = 4000 (grad_b's reduction, 62.5 stages) and n = 4040 (grad_a's, 63.1 stages) at full width
    M, N, K = 4000, 4040, 4096
    a, b, g = inputs(M, N, K, 4242)
    ga, gb = run(a, b, g)
    rng = np.random.default_rng(4243)
    ra, ca = rng.integers(0, M, 2048), rng.integers(0, K, 2048)
    rb, cb = rng.integers(0, K, 2048), rng.integers(0, N, 2048)
    (pa, ta), (pb, tb) = gemm_bwd_at(a, b, g, ra, ca, rb, cb)
    for name, x, y, t in (("grad_a", ga[ra, ca], pa, ta), ("grad_b", gb[rb, cb], pb, tb)):
        bad, ratio = compare.excess(x, y, compare.f16_tolerance(y, t))
        assert bad == 0, f"{name}: {bad} outside tolerance, max ratio {ratio:.3f}"


def test_config_4096_sampled():
    cfg = workloads.GEMM_4096
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    a, b, g = inputs(M, N, K, cfg["seed"])
    ga, gb = run(a, b, g)
    rng = np.random.default_rng(cfg["check_seed"])
    ra, ca = rng.integers(0, M, 2048), rng.integers(0, K, 2048)
    rb, cb = rng.integers(0, K, 2048), rng.integers(0, N, 2048)
    (pa, ta), (pb, tb) = gemm_bwd_at(a, b, g, ra, ca, rb, cb)
    for name, x, y, t in (("grad_a", ga[ra, ca], pa, ta), ("grad_b", gb[rb, cb], pb, tb)):
        bad, ratio = compare.excess(x, y, compare.f16_tolerance(y, t))
        assert bad == 0, f"{name}: {bad} outside tolerance, max ratio {ratio:.3f}"


def test_empty_problems():
    # k == 0: both gradients empty, nothing launched
    a = torch.empty((3, 0), dtype=torch.float16, device=DEV)
    b = torch.empty((0, 5), dtype=torch.float16, device=DEV)
    g = torch.zeros((3, 5), dtype=torch.float32, device=DEV)
    ga, gb = kaio.kaio_gemm_f16f32_bwd(a, b, g)
    assert ga.shape == (3, 0) and gb.shape == (0, 5)
    # m == 0: grad_b is the empty sum
    a = torch.empty((0, 6), dtype=torch.float16, device=DEV)
    b = torch.ones((6, 5), dtype=torch.float16, device=DEV)
    g = torch.empty((0, 5), dtype=torch.float32, device=DEV)
    gb = torch.full((6, 5), float("nan"), dtype=torch.float16, device=DEV)
    kaio.kaio_gemm_f16f32_bwd(a, b, g, grad_b=gb)
    torch.cuda.synchronize()
    assert (gb == 0).all()
    # n == 0: grad_a is the empty sum
    a = torch.ones((4, 6), dtype=torch.float16, device=DEV)
    b = torch.empty((6, 0), dtype=torch.float16, device=DEV)
    g = torch.empty((4, 0), dtype=torch.float32, device=DEV)
    ga = torch.full((4, 6), float("nan"), dtype=torch.float16, device=DEV)
    kaio.kaio_gemm_f16f32_bwd(a, b, g, grad_a=ga)
    torch.cuda.synchronize()
    assert (ga == 0).all()

