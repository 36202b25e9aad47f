"""Launch semantics on the GPU: caller streams, HIP graph capture and replay, determinism.

Every entry point launches asynchronously on the stream it is given and allocates
nothing, so it can be recorded into a HIP graph.  These tests check that:
* work issued on a side stream gives bit-identical results to the default stream;
* a captured graph, replayed several times with new input contents written in
  place (and other eager work) between replays, recomputes every output from the
  inputs of that replay, matching an eager call bit for bit;
* repeated calls are bit-identical and leave their inputs untouched.
The eager results themselves are checked against the oracle in the other GPU tests;
here the first result of each kind is also checked, so a wrong-but-stable kernel
cannot pass.
"""
import numpy as np
import pytest
import torch

import int4_group_quantized_w4a16_amd as kaio
from int4_group_quantized_w4a16_amd import workloads
from oracle import compare
from oracle.dequant_bwd import dequant_bwd
from oracle.gemm import gemm
from oracle.gemm_bwd import gemm_bwd
from oracle.qkv import qkv_project
from tests.gpu_util import DEV, to_dev, to_host

pytestmark = pytest.mark.gpu


def bits(t):
    return to_host(t).view(np.uint16 if t.element_size() == 2 else np.uint32).copy()


def qkv_case(M, N, K, seed):
    inp = workloads.qkv_inputs(M, N, K, seed)
    return inp, to_dev(inp.x), [to_dev(a) for a in inp.w], [to_dev(a) for a in inp.s]


def check_qkv(outs, inp):
    ys, ts = qkv_project(inp.x, inp.w, inp.s)
    for o, y, t in zip(outs, ys, ts):
        bad, ratio = compare.excess(to_host(o), y, compare.qkv_tolerance(y, t))
        assert bad == 0, f"{bad} outside tolerance (max ratio {ratio:.3f})"


# split-K kernel with 8 and 16 x rows kept, with two row tiles per wave (m = 24), then the tile
# kernel with one output per workgroup (four sets at m = 40, two at m = 100) and with three
@pytest.mark.parametrize("M", [5, 12, 24, 40, 100, 200])
def test_qkv_side_stream_matches_default_stream(M):
    inp, x, w, s = qkv_case(M, 264, 512, 31 + M)
    ref = kaio.kaio_qkv_w4a16(x, *w, *s)
    torch.cuda.synchronize()
    check_qkv(ref, inp)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        outs = [torch.full_like(r, float("nan")) for r in ref]
        kaio.kaio_qkv_w4a16(x, *w, *s, *outs)          # current stream = side
    side.synchronize()
    for a, b in zip(ref, outs):
        assert np.array_equal(bits(a), bits(b))


def replay_and_compare(graph, refill, eager, outs):
    """Replay `graph` three times; before each replay `refill(i)` rewrites the
    inputs in place; after it the outputs must equal `eager()` bit for bit."""
    for i in range(3):
        refill(i)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [bits(o) for o in outs]
        want = [bits(o) for o in eager()]
        for a, b in zip(got, want):
            assert np.array_equal(a, b), f"replay {i} differs from the eager call"
        # unrelated eager work between replays
        torch.randn(1024, device=DEV).sum().item()


def capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                      # warm-up outside the graph (library load, attributes)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


# K = 4096 at M = 8 gives every split-K wave exactly two groups (its straight-line path); M = 300
# runs the tile kernel with one set of waves (K = 384: 3 groups) and with two (K = 512)
@pytest.mark.parametrize("M,K", [(8, 384), (8, 4096), (24, 512), (40, 1024), (100, 640), (300, 384), (300, 512)])
def test_qkv_graph_replay_uses_current_inputs(M, K):
    N = 136
    inp, x, w, s = qkv_case(M, N, K, 7)
    outs = [torch.empty((M, N), dtype=torch.float16, device=DEV) for _ in range(3)]
    g = capture(lambda: kaio.kaio_qkv_w4a16(x, *w, *s, *outs))
    rng = np.random.default_rng(3)

    def refill(i):
        if i == 0:
            return
        x.copy_(torch.from_numpy(rng.standard_normal((M, K)).astype(np.float16)))
        w[i % 3].copy_(torch.from_numpy(rng.integers(-2 ** 31, 2 ** 31, size=(K // 8, N), dtype=np.int64)
                                        .astype(np.int32)))
        for o in outs:
            o.fill_(float("nan"))
    replay_and_compare(g, refill, lambda: kaio.kaio_qkv_w4a16(x, *w, *s), outs)


def test_gemm_graph_replay_and_determinism():
    M, N, K = 300, 264, 192           # the direct-to-LDS path with ragged m and n
    a_np, b_np = workloads.gemm_inputs(M, N, K, seed=77)
    a, b = to_dev(a_np), to_dev(b_np)
    a0, b0 = a.clone(), b.clone()
    c = torch.empty((M, N), dtype=torch.float32, device=DEV)
    first = kaio.kaio_gemm_f16f32(a, b)
    torch.cuda.synchronize()
    cref, t = gemm(a_np, b_np)
    bad, ratio = compare.excess(to_host(first), cref, compare.gemm_tolerance(t))
    assert bad == 0, f"{bad} outside tolerance (max ratio {ratio:.3f})"
    again = kaio.kaio_gemm_f16f32(a, b)
    torch.cuda.synchronize()
    assert np.array_equal(bits(first), bits(again))
    assert torch.equal(a, a0) and torch.equal(b, b0)

    g = capture(lambda: kaio.kaio_gemm_f16f32(a, b, c))
    rng = np.random.default_rng(5)

    def refill(i):
        a.copy_(torch.from_numpy(rng.standard_normal((M, K)).astype(np.float16)))
        c.fill_(float("nan"))
    replay_and_compare(g, refill, lambda: [kaio.kaio_gemm_f16f32(a, b)], [c])


def test_gemm_empty_reduction_in_graph():
    # k == 0 writes zeros with a fill kernel (no memset node in the graph)
    a = torch.empty((33, 0), dtype=torch.float16, device=DEV)
    b = torch.empty((0, 17), dtype=torch.float16, device=DEV)
    c = torch.full((33, 17), float("nan"), dtype=torch.float32, device=DEV)
    g = capture(lambda: kaio.kaio_gemm_f16f32(a, b, c))
    for _ in range(3):
        c.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert (c == 0).all()


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_dequant_bwd_graph_replay_and_determinism(dt):
    outer, axis, group = 96, 1024, 128
    dy_np, sc_np = workloads.dequant_bwd_inputs(outer, axis, group, 11, dt)
    dy, sc = to_dev(dy_np), to_dev(sc_np)
    dy0, sc0 = dy.clone(), sc.clone()
    first = kaio.kaio_dequant_group_bwd(dy, sc, group)
    torch.cuda.synchronize()
    want = dequant_bwd(dy_np, sc_np, group, dt)
    assert np.array_equal(bits(first), want.view(np.uint16 if dt == "bf16" else np.uint32))
    again = kaio.kaio_dequant_group_bwd(dy, sc, group)
    torch.cuda.synchronize()
    assert np.array_equal(bits(first), bits(again))
    assert torch.equal(dy, dy0) and torch.equal(sc, sc0)

    dq = torch.empty_like(dy)
    g = capture(lambda: kaio.kaio_dequant_group_bwd(dy, sc, group, dq))

    def refill(i):
        new, _ = workloads.dequant_bwd_inputs(outer, axis, group, 100 + i, dt)
        dy.copy_(to_dev(new))
        dq.zero_()
    replay_and_compare(g, refill, lambda: [kaio.kaio_dequant_group_bwd(dy, sc, group)], [dq])


def test_gemm_bwd_graph_replay_and_determinism():
    M, N, K = 192, 256, 320            # both gradients on the direct-to-LDS path
    a_np, b_np = workloads.gemm_inputs(M, N, K, seed=78)
    rng = np.random.default_rng(6)
    a, b = to_dev(a_np), to_dev(b_np)
    grad = to_dev(rng.standard_normal((M, N)).astype(np.float32))
    ins0 = [t.clone() for t in (a, b, grad)]
    first = kaio.kaio_gemm_f16f32_bwd(a, b, grad)
    torch.cuda.synchronize()
    (da, ta), (db, tb) = gemm_bwd(a_np, b_np, to_host(grad))
    for o, y, t in zip(first, (da, db), (ta, tb)):
        bad, ratio = compare.excess(to_host(o), y, compare.f16_tolerance(y, t))
        assert bad == 0, f"{bad} outside tolerance (max ratio {ratio:.3f})"
    again = kaio.kaio_gemm_f16f32_bwd(a, b, grad)
    torch.cuda.synchronize()
    for x, y in zip(first, again):
        assert np.array_equal(bits(x), bits(y))
    assert all(torch.equal(x, y) for x, y in zip((a, b, grad), ins0))

    ga = torch.empty((M, K), dtype=torch.float16, device=DEV)
    gb = torch.empty((K, N), dtype=torch.float16, device=DEV)
    ws = torch.empty((M * N * 2,), dtype=torch.uint8, device=DEV)
    g = capture(lambda: kaio.kaio_gemm_f16f32_bwd(a, b, grad, ga, gb, ws))

    def refill(i):
        grad.copy_(torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32)))
        ws.fill_(0xff)
        ga.fill_(float("nan"))
        gb.fill_(float("nan"))
    replay_and_compare(g, refill, lambda: list(kaio.kaio_gemm_f16f32_bwd(a, b, grad)), [ga, gb])
