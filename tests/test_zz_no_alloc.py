"""Allocation-free GEMM backward (kaio_gemm_f16f32_bwd_noalloc) on the GPU.

The entry point stages f16(grad) in the library's static per-device buffer
instead of a caller workspace.  It is called here through the C ABI and
compared, bit for bit, with kaio_gemm_f16f32_bwd (caller workspace) on the
same inputs -- two calls in a row, the second on a smaller problem, so the
second call reads a buffer that still holds the first call's contents.  The
first pair is also checked against the oracle.
"""
import ctypes

import numpy as np
import pytest
import torch

import int4_group_quantized_w4a16_amd as kaio
from int4_group_quantized_w4a16_amd import workloads
from oracle import compare
from oracle.gemm_bwd import gemm_bwd
from tests.gpu_util import DEV, to_dev, to_host

pytestmark = pytest.mark.gpu


def inputs(m, n, k, seed):
    a, b = workloads.gemm_inputs(m, n, k, seed)
    g = np.random.default_rng(seed + 1).standard_normal((m, n)).astype(np.float32)
    return a, b, g


def noalloc(a, b, g):
    M, K = a.shape
    N = b.shape[1]
    ga = torch.full((M, K), float("nan"), dtype=torch.float16, device=DEV)
    gb = torch.full((K, N), float("nan"), dtype=torch.float16, device=DEV)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = kaio.lib().kaio_gemm_f16f32_bwd_noalloc(a.data_ptr(), b.data_ptr(), g.data_ptr(), ga.data_ptr(),
                                                 gb.data_ptr(), M, N, K, stream)
    assert st == 0, kaio.kaio_last_error()
    return ga, gb


def with_workspace(a, b, g):
    ga, gb = kaio.kaio_gemm_f16f32_bwd(a, b, g)
    return ga, gb


def bits(t):
    return to_host(t).view(np.uint16)


# first call: the direct-to-LDS path for both gradients; second, smaller: the any-shape
# fallback for grad_b (m % 64 != 0) and the direct path for grad_a
@pytest.mark.parametrize("shapes", [((512, 384, 320), (200, 136, 128)),
                                    ((1024, 1024, 512), (64, 64, 64))])
def test_noalloc_matches_workspace_entry_point(shapes):
    for i, (m, n, k) in enumerate(shapes):
        a_np, b_np, g_np = inputs(m, n, k, seed=31 * m + n + k)
        a, b, g = to_dev(a_np), to_dev(b_np), to_dev(g_np)
        got = noalloc(a, b, g)
        torch.cuda.synchronize()
        want = with_workspace(a, b, g)
        torch.cuda.synchronize()
        for x, y in zip(got, want):
            assert np.array_equal(bits(x), bits(y)), f"call {i} ({m}x{n}x{k}) differs from the workspace entry point"
        if i == 0:
            (da, ta), (db, tb) = gemm_bwd(a_np, b_np, g_np)
            for x, y, t in ((got[0], da, ta), (got[1], db, tb)):
                bad, ratio = compare.excess(to_host(x), y, compare.f16_tolerance(y, t))
                assert bad == 0, f"{bad} outside tolerance (max ratio {ratio:.3f})"


def test_noalloc_rejects_problems_beyond_its_buffer():
    L = kaio.lib()
    # m * n * 2 = 64 MiB + 2 * 4096 bytes: one row more than the buffer holds; nothing is launched
    st = L.kaio_gemm_f16f32_bwd_noalloc(0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 8193, 4096, 64, None)
    assert st == 3 and "static buffer" in kaio.kaio_last_error()
