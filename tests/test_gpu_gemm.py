"""Dense f16 x f16 -> f32 GEMM on the GPU against the CPU oracle (through the C ABI).
Tolerance: |c - C*| <= 1e-5 * sum_k |a_ik * b_kj|; exact cases bit for bit."""
import numpy as np
import pytest
import torch

import int4_group_quantized_w4a16_amd as kaio
from int4_group_quantized_w4a16_amd import workloads
from oracle import compare
from oracle.gemm import gemm, gemm_at
from tests.conftest import load_golden
from tests.gpu_util import DEV, to_dev, to_host

pytestmark = pytest.mark.gpu


def run(a, b):
    c = kaio.kaio_gemm_f16f32(to_dev(a), to_dev(b))
    torch.cuda.synchronize()
    return to_host(c)


def test_golden_handworked_bitwise():
    for case in load_golden("gemm_handworked.json")["cases"]:
        a = np.array(case["a"], dtype=np.float16)
        b = np.array(case["b"], dtype=np.float16)
        assert np.array_equal(run(a, b), np.array(case["c"], dtype=np.float32))


def test_identity_and_exact_integers():
    rng = np.random.default_rng(1)
    a = rng.standard_normal((64, 96)).astype(np.float16)
    assert np.array_equal(run(a, np.eye(96, dtype=np.float16)), a.astype(np.float32))
    for n in (260, 264):   # 264: the direct-to-LDS path
        ai = rng.integers(-8, 9, size=(300, 1024)).astype(np.float16)
        bi = rng.integers(-8, 9, size=(1024, n)).astype(np.float16)
        c, _ = gemm(ai, bi)
        assert np.array_equal(run(ai, bi), c.astype(np.float32))


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (300, 200, 100), (257, 259, 72), (100, 100, 4096),
                                   (513, 300, 520), (16, 1000, 33), (256, 256, 64),
                                   # k % 64 == 0 and n % 8 == 0: the direct-to-LDS path, ragged m and n
                                   (300, 264, 128), (513, 136, 192), (40, 520, 64), (257, 8, 256),
                                   # k % 8 == 0, k % 64 != 0: the direct-to-LDS path with a ragged last stage
                                   (300, 264, 200), (257, 136, 72), (64, 64, 8), (1, 8, 8), (513, 520, 4104),
                                   (40, 1024, 4000),
                                   # n and k both off multiples of 8 (both operands on clamped 16-byte
                                   # chunk loads), down to a reduction of one partial chunk
                                   (300, 259, 100), (70, 1001, 515), (33, 17, 9), (9, 8, 11)])
def test_ragged_shapes(M, N, K):
    a, b = workloads.gemm_inputs(M, N, K, seed=M + N + K)
    c, t = gemm(a, b)
    bad, ratio = compare.excess(run(a, b), c, compare.gemm_tolerance(t))
    assert bad == 0, f"{bad} outside tolerance, max ratio {ratio:.3f}"


def test_empty_reduction_writes_zeros():
    c = torch.full((33, 17), float("nan"), dtype=torch.float32, device=DEV)
    kaio.kaio_gemm_f16f32(torch.empty((33, 0), dtype=torch.float16, device=DEV),
                          torch.empty((0, 17), dtype=torch.float16, device=DEV), c)
    torch.cuda.synchronize()
    assert (c == 0).all()


def test_config_4096_sampled():
    cfg = workloads.GEMM_4096
    a, b = workloads.gemm_inputs(cfg["M"], cfg["N"], cfg["K"], cfg["seed"])
    got = run(a, b)
    rows, cols = workloads.gemm_check_positions(cfg["M"], cfg["N"], 4096, cfg["check_seed"])
    c, t = gemm_at(a, b, rows, cols)
    bad, ratio = compare.excess(got[rows, cols], c, compare.gemm_tolerance(t))
    assert bad == 0, f"{bad} outside tolerance, max ratio {ratio:.3f}"
    print(f"gemm 4096^3 ({rows.size} entries): max |d|/tol = {ratio:.4f}")
    assert np.array_equal(run(a, b), got)          # run-to-run identical


@pytest.mark.parametrize("M,N,K", [(200, 136, 72), (64, 256, 4040)])
def test_ragged_reduction_exact_integers_bitwise(M, N, K):
    # small integers: every partial sum is exact in f32, so the ragged last stage (k % 64 != 0)
    # must reproduce the exact product bit for bit -- the chunks past k read as zeros
    rng = np.random.default_rng(M + K)
    a = rng.integers(-4, 5, size=(M, K)).astype(np.float16)
    b = rng.integers(-4, 5, size=(K, N)).astype(np.float16)
    c, _ = gemm(a, b)
    assert np.array_equal(run(a, b), c.astype(np.float32))


@pytest.mark.parametrize("M,N,K", [(300, 264, 256), (257, 259, 72)])
def test_non_finite_inputs_stay_in_their_rows_and_columns(M, N, K):
    # IEEE propagation: NaN in A row 3 -> C row 3 NaN; +inf in B column 7 at k0 -> column 7 is
    # +-inf by the sign of A[:, k0] (NaN where it is 0 or where row 3's NaN meets it); the rest of
    # C is finite and matches the oracle (the direct-load path and the register-staged fallback).
    a, b = workloads.gemm_inputs(M, N, K, 41 + M)
    k0 = 5
    a[:, k0] = np.where(np.arange(M) % 5 == 0, np.float16(0), a[:, k0])
    a[3, 11] = np.float16(np.nan)
    b[k0, 7] = np.float16(np.inf)
    c = run(a, b)
    assert np.isnan(c[3]).all()
    rows = np.array([r for r in range(M) if r != 3])
    col7 = c[rows, 7]
    ak = a[rows, k0].astype(np.float64)
    assert np.array_equal(np.isnan(col7), ak == 0)
    assert np.array_equal(np.sign(col7[ak != 0]), np.sign(ak[ak != 0]).astype(np.float32))
    cols = np.array([j for j in range(N) if j != 7])
    a2, b2 = a[rows], b[:, cols]
    ref, t = gemm(a2, b2)
    bad, ratio = compare.excess(c[np.ix_(rows, cols)], ref, compare.gemm_tolerance(t))
    assert bad == 0, f"{bad} finite outputs outside tolerance, max |d|/tol = {ratio:.3f}"
