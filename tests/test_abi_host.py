"""C-ABI boundary on the host: the library loads, exports every declared entry
point, and rejects every invalid call before touching a device.

Pointers here are fake addresses that are never dereferenced: each call is
built to fail validation, or (without a GPU) the device check.  Tests that
would pass validation are skipped when a GPU is visible.
"""
import ctypes
import os
import re

import pytest

import int4_group_quantized_w4a16_amd as kaio

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "kaio.h")
OK, ARG, PROB, UNSUP, DEVICE = 0, 1, 2, 3, 4
A = 0x100000          # a fake, 16-byte aligned device address
STEP = 0x10000000     # spacing that keeps fake buffers disjoint


def gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


no_gpu_only = pytest.mark.skipif(gpu_visible(), reason="fake pointers would reach a real launch")


def declared_functions(header=HEADER):
    src = open(header).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kaio_[a-z0-9_]+)\s*\(", src)))


def test_measurement_library_exports_its_header():
    # libkaio_roof.so: the benchmark's plain-read, strip-read, MFMA-alone and clock-probe kernels
    # (not libkaio's ABI)
    header = os.path.join(os.path.dirname(HEADER), "kaio_roof.h")
    names = declared_functions(header)
    assert set(names) == {"kaio_roof_stream_read", "kaio_roof_sink_bytes", "kaio_roof_clock_probe",
                          "kaio_roof_wall_clock_khz", "kaio_roof_strip_read", "kaio_roof_strip_sink_bytes",
                          "kaio_roof_mfma", "kaio_roof_mfma_flops"}
    L = ctypes.CDLL(os.path.join(os.path.dirname(os.path.abspath(kaio.__file__)), "libkaio_roof.so"))
    for n in names:
        assert hasattr(L, n), n
    L.kaio_roof_sink_bytes.restype = ctypes.c_size_t
    L.kaio_roof_sink_bytes.argtypes = [ctypes.c_size_t, ctypes.c_int, ctypes.c_int]
    assert L.kaio_roof_sink_bytes(16 * 256 * 4 * 3 + 16, 4, 256) == 4 * 256 * 4
    L.kaio_roof_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_void_p]
    assert L.kaio_roof_stream_read(A, 100, A + STEP, 4, 256, None) == 1      # not a multiple of 16
    assert L.kaio_roof_stream_read(A, 1024, A + STEP, 3, 256, None) == 2     # unsupported shape
    L.kaio_roof_strip_sink_bytes.restype = ctypes.c_size_t
    L.kaio_roof_strip_sink_bytes.argtypes = [ctypes.c_uint, ctypes.c_int]
    assert L.kaio_roof_strip_sink_bytes(4096, 64) == 3 * 64 * 1024 * 4
    assert L.kaio_roof_strip_sink_bytes(4096, 16) == 256 * 512 * 4
    L.kaio_roof_strip_read.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_uint, ctypes.c_uint, ctypes.c_int,
                                                               ctypes.c_void_p, ctypes.c_void_p]
    # validation happens before any launch: no GPU needed
    assert L.kaio_roof_strip_read(A, A + STEP, A + 2 * STEP, 100, 4096, 64, A + 3 * STEP, None) == 1  # rows % 128
    assert L.kaio_roof_strip_read(A, A + STEP, A + 2 * STEP, 512, 4000, 64, A + 3 * STEP, None) == 1  # cols % 64
    assert L.kaio_roof_strip_read(A, None, A + 2 * STEP, 512, 4096, 64, A + 3 * STEP, None) == 1      # null array
    L.kaio_roof_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    L.kaio_roof_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    L.kaio_roof_mfma_flops.restype = ctypes.c_double
    assert L.kaio_roof_mfma_flops(256, 2048) == 2048 * 4 * 256 * 8 * 2 * 16 * 16 * 32
    assert L.kaio_roof_mfma(None, 256, 2048, None) == 1          # null sink
    assert L.kaio_roof_mfma(A, 6, 2048, None) == 1               # iterations not a multiple of 4
    assert L.kaio_roof_mfma(A, 256, 0, None) == 1                # no workgroups


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) >= {"kaio_qkv_w4a16", "kaio_gemm_f16f32", "kaio_dequant_group_bwd", "kaio_last_error"}
    L = ctypes.CDLL(kaio.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert kaio.kaio_version().startswith("kaio-mi355x")


def qkv(x=A, w=(A + STEP, A + 2 * STEP, A + 3 * STEP), s=(A + 4 * STEP, A + 5 * STEP, A + 6 * STEP),
        o=(A + 7 * STEP, A + 8 * STEP, A + 9 * STEP), m=4, n=64, k=256, g=128):
    st = kaio.lib().kaio_qkv_w4a16(x, *w, *s, *o, m, n, k, g, None)
    return st, kaio.kaio_last_error()


def test_qkv_w8a16_validation():
    L = kaio.lib()
    w = (A + STEP, A + 2 * STEP, A + 3 * STEP)
    s = (A + 4 * STEP, A + 5 * STEP, A + 6 * STEP)
    o = (A + 7 * STEP, A + 8 * STEP, A + 9 * STEP)
    call = lambda **kw: (L.kaio_qkv_w8a16(kw.get("x", A), *kw.get("w", w), *s, *kw.get("o", o), kw.get("m", 4),
                                          64, kw.get("k", 256), kw.get("g", 128), None), kaio.kaio_last_error())
    st, msg = call(g=64)
    assert st == UNSUP and msg.startswith("kaio::qkv_w8a16:") and "group_size" in msg
    assert call(k=200)[0] == PROB
    assert call(m=0)[0] == OK
    assert "output q is null" in call(o=(0, o[1], o[2]))[1]
    # the packed weights are k/4 rows x 64 columns x 4 bytes = 16 KiB at k = 256: a weight
    # tensor starting 8 KiB into another overlaps it for W8A16 (it would not for INT4's 8 KiB)
    assert call(o=(A + STEP + 8192, o[1], o[2]))[1].endswith("overlaps w_q_packed")


def test_qkv_validation_order_and_messages():
    st, msg = qkv(g=64)
    assert st == UNSUP and msg.startswith("kaio::qkv_w4a16:") and "group_size" in msg
    st, msg = qkv(k=200)
    assert st == PROB and "multiple of group_size" in msg
    st, msg = qkv(k=64)
    assert st == PROB
    assert qkv(m=0)[0] == OK and qkv(n=0)[0] == OK
    assert qkv(m=0, o=(0, 0, 0))[0] == OK                       # empty: pointers not needed
    st, msg = qkv(o=(0, A + 8 * STEP, A + 9 * STEP))
    assert st == ARG and "output q is null" in msg
    st, msg = qkv(x=0)
    assert st == ARG and "input x is null" in msg
    st, msg = qkv(w=(A + STEP, 0, A + 3 * STEP))
    assert st == ARG and "w_k_packed" in msg
    st, msg = qkv(s=(A + 4 * STEP, A + 5 * STEP, 0))
    assert st == ARG and "scales_v" in msg
    st, msg = qkv(x=A + 8)
    assert st == ARG and "aligned" in msg
    st, msg = qkv(o=(A + 7 * STEP, A + 7 * STEP, A + 9 * STEP))
    assert st == ARG and "overlaps" in msg
    st, msg = qkv(o=(A + 96, A + 8 * STEP, A + 9 * STEP))       # q inside x (x is 4*256*2 bytes)
    assert st == ARG and "overlaps x" in msg
    st, msg = qkv(m=2 ** 32 - 1, n=2 ** 32 - 1)
    assert st == PROB and "too large" in msg
    # the documented per-dimension limits (32-bit per-lane byte offsets in the kernels)
    assert qkv(m=16, n=2 ** 26, k=128)[0] == PROB
    assert qkv(m=16, n=8, k=2 ** 24)[0] == PROB


@no_gpu_only
def test_qkv_valid_call_without_gpu_reports_device():
    st, msg = qkv()
    assert st == DEVICE and "no CPU fallback" in msg
    st, _ = qkv(k=0)            # k == 0 writes zeros: still needs the device
    assert st == DEVICE


def gemm(a=A, b=A + STEP, c=A + 2 * STEP, m=8, n=8, k=8):
    return kaio.lib().kaio_gemm_f16f32(a, b, c, m, n, k, None), kaio.kaio_last_error()


def test_gemm_validation():
    assert gemm(m=0)[0] == OK and gemm(n=0, c=0)[0] == OK
    st, msg = gemm(c=0)
    assert st == ARG and msg.startswith("kaio::gemm_f16f32:") and "output c is null" in msg
    assert gemm(a=0)[0] == ARG and gemm(b=0)[0] == ARG
    assert gemm(c=A + 2 * STEP + 4)[0] == ARG
    st, msg = gemm(c=A + 64)
    assert st == ARG and "overlaps a" in msg
    st, msg = gemm(m=2 ** 32 - 1, n=2 ** 32 - 1)
    assert st == PROB


@no_gpu_only
def test_gemm_without_gpu_reports_device():
    assert gemm()[0] == DEVICE
    assert gemm(a=0, b=0, k=0)[0] == DEVICE   # k == 0: inputs unused, zeros still need the device


def gbwd(a=A, b=A + STEP, g=A + 2 * STEP, ga=A + 3 * STEP, gb=A + 4 * STEP, m=64, n=64, k=64,
         ws=A + 5 * STEP, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = kaio.lib().kaio_gemm_f16f32_bwd_workspace_size(m, n)
    st = kaio.lib().kaio_gemm_f16f32_bwd(a, b, g, ga, gb, m, n, k, ws, ws_bytes, None)
    return st, kaio.kaio_last_error()


def test_gemm_bwd_validation():
    L = kaio.lib()
    assert L.kaio_gemm_f16f32_bwd_workspace_size(300, 72) == 300 * 72 * 2
    assert gbwd(k=0, a=0, b=0, g=0, ga=0, gb=0, ws=0)[0] == OK        # both gradients empty
    st, msg = gbwd(ga=0)
    assert st == ARG and msg.startswith("kaio::gemm_f16f32_bwd:") and "grad_a is null" in msg
    assert "grad_b is null" in gbwd(gb=0)[1]
    for kw, text in ((dict(a=0), "input a"), (dict(b=0), "input b"), (dict(g=0), "input grad"),
                     (dict(ws=0), "workspace is null")):
        st, msg = gbwd(**kw)
        assert st == ARG and text in msg, (kw, msg)
    st, msg = gbwd(ws_bytes=64 * 64 * 2 - 1)
    assert st == ARG and "workspace_bytes" in msg
    assert gbwd(gb=A + 4 * STEP + 8)[0] == ARG
    assert "not 16-byte aligned" in gbwd(ws=A + 5 * STEP + 4)[1]
    assert "grad_a overlaps grad" in gbwd(ga=A + 2 * STEP + 64)[1]
    assert "grad_a overlaps workspace" in gbwd(ws=A + 3 * STEP + 4096)[1]
    assert "grad_b overlaps workspace" in gbwd(ws=A + 4 * STEP)[1]
    assert "workspace overlaps a" in gbwd(ws=A + 16)[1]
    assert gbwd(m=2 ** 32 - 1, n=2 ** 32 - 1)[0] == PROB
    # m == 0 or n == 0: inputs and workspace are unused, only the written gradient is checked
    assert gbwd(m=0, a=0, b=0, g=0, ws=0, ga=0)[0] in (OK, DEVICE)
    assert gbwd(n=0, a=0, b=0, g=0, ws=0, gb=0)[0] in (OK, DEVICE)


@no_gpu_only
def test_gemm_bwd_without_gpu_reports_device():
    assert gbwd()[0] == DEVICE
    assert gbwd(m=0, a=0, b=0, g=0, ws=0, ga=0)[0] == DEVICE   # zeros for grad_b need the device


def gbwd_noalloc(a=A, b=A + STEP, g=A + 2 * STEP, ga=A + 3 * STEP, gb=A + 4 * STEP, m=64, n=64, k=64):
    st = kaio.lib().kaio_gemm_f16f32_bwd_noalloc(a, b, g, ga, gb, m, n, k, None)
    return st, kaio.kaio_last_error()


def test_gemm_bwd_noalloc_validation():
    # limit of the static f16(grad) buffer: 64 MiB = 2^25 halves
    st, msg = gbwd_noalloc(m=8193, n=4096)
    assert st == UNSUP and msg.startswith("kaio::gemm_f16f32_bwd_noalloc:") and "static buffer" in msg
    assert gbwd_noalloc(m=2 ** 32 - 1, n=2 ** 32 - 1)[0] == PROB          # size check first
    assert gbwd_noalloc(k=0, a=0, b=0, g=0, ga=0, gb=0)[0] == OK
    assert "grad_a is null" in gbwd_noalloc(ga=0)[1]
    assert "input grad is null" in gbwd_noalloc(g=0)[1]
    assert "not 16-byte aligned" in gbwd_noalloc(gb=A + 4 * STEP + 8)[1]
    assert "grad_a overlaps grad" in gbwd_noalloc(ga=A + 2 * STEP + 64)[1]


@no_gpu_only
def test_gemm_bwd_noalloc_without_gpu_reports_device():
    assert gbwd_noalloc()[0] == DEVICE
    assert gbwd_noalloc(m=8192, n=4096)[0] == DEVICE   # exactly the buffer size is accepted


def bwd(dt=0, outer=4, axis=256, g=128, dy=A, sc=A + STEP, dq=A + 2 * STEP):
    return kaio.lib().kaio_dequant_group_bwd(dt, outer, axis, g, dy, sc, dq, None, 0, None), kaio.kaio_last_error()


def test_dequant_validation():
    st, msg = bwd(dt=7)
    assert st == UNSUP and msg.startswith("kaio::dequant_group_bwd:")
    assert bwd(outer=-1)[0] == PROB and bwd(axis=-128)[0] == PROB
    st, msg = bwd(g=0)
    assert st == PROB and "group_size" in msg
    assert bwd(g=-4)[0] == PROB
    st, msg = bwd(axis=200, g=128)
    assert st == PROB and "multiple" in msg
    assert bwd(outer=0, dy=0, sc=0, dq=0)[0] == OK
    assert bwd(axis=0, dy=0, sc=0, dq=0)[0] == OK
    assert bwd(dy=0)[0] == ARG and bwd(sc=0)[0] == ARG and bwd(dq=0)[0] == ARG
    st, msg = bwd(dt=0, dy=A + 2)
    assert st == ARG and "aligned" in msg
    st, msg = bwd(dq=A + 64)
    assert st == ARG and "overlaps d_output" in msg
    st, msg = bwd(dq=A + STEP + 8)
    assert st == ARG and "overlaps scale" in msg


@no_gpu_only
def test_dequant_without_gpu_reports_device():
    for dt in (0, 1, 2, 3):
        assert bwd(dt=dt)[0] == DEVICE
    assert bwd(dt=1, dy=A + 2, dq=A + 2 * STEP + 2)[0] == DEVICE   # element-aligned bf16 is accepted


def test_last_error_is_per_thread_and_cleared_on_success():
    import threading
    qkv(g=64)
    assert "group_size" in kaio.kaio_last_error()
    seen = []
    th = threading.Thread(target=lambda: seen.append(kaio.kaio_last_error()))
    th.start(); th.join()
    assert seen == [""]
    assert qkv(m=0)[0] == OK and kaio.kaio_last_error() == ""


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 128, dtype=torch.float16)
    w = torch.zeros(16, 8, dtype=torch.int32)
    s = torch.zeros(1, 8, dtype=torch.float16)
    with pytest.raises(ValueError, match="no CPU fallback"):
        kaio.kaio_qkv_w4a16(x, w, w, w, s, s, s)
    with pytest.raises(ValueError, match="no CPU fallback"):
        kaio.kaio_gemm_f16f32(torch.zeros(2, 2, dtype=torch.float16), torch.zeros(2, 2, dtype=torch.float16))
    with pytest.raises(ValueError, match="no CPU fallback"):
        kaio.kaio_dequant_group_bwd(torch.zeros(2, 4), torch.zeros(2, 1), 4)


def test_qkv_plan_validation_and_forms():
    L = kaio.lib()
    plan = (ctypes.c_uint32 * 5)()
    assert L.kaio_qkv_plan(256, 64, 256, 5, plan) == 1 and "bits" in kaio.kaio_last_error()
    assert L.kaio_qkv_plan(256, 64, 256, 4, None) == 1 and "plan is null" in kaio.kaio_last_error()
    assert L.kaio_qkv_plan(256, 64, 200, 4, plan) == 2 and "multiple of group_size" in kaio.kaio_last_error()
    assert L.kaio_qkv_plan(0, 64, 256, 4, plan) == 0 and list(plan) == [0, 0, 0, 0, 0]
    # m <= 32, and m <= 64 where the four-set tile form does not apply (INT8, or a group count
    # not divisible by 4): the split-K kernel, 3 outputs x strips
    for m, k, bits in ((8, 4096, 4), (32, 4096, 4), (64, 4096, 8), (64, 384, 4), (40, 640, 4)):
        p = kaio.kaio_qkv_plan(m, 4096, k, bits)
        assert p["kernel"] == "split_k" and p["workgroups"] == 3 * 4096 // p["rows"], (m, k, bits)
    # INT4, 32 < m <= 64, k / 128 divisible by 4: one output per workgroup, 64-row tiles, four sets
    for m in (33, 64):
        p = kaio.kaio_qkv_plan(m, 4096, 4096)
        assert p["kernel"] == "tile_one_output" and (p["waves"], p["rows"], p["sets"]) == (4, 64, 4)
        assert p["workgroups"] == 3 * 4096 // 64
    # 64 < m <= 128: the tile kernel with one output per workgroup, 96-row tiles up to 96 rows,
    # two sets when the group count is even
    for m, k, rows, sets in ((65, 4096, 96, 2), (96, 4224, 96, 1), (97, 4096, 128, 2), (128, 384, 128, 1)):
        p = kaio.kaio_qkv_plan(m, 4096, k)
        assert p["kernel"] == "tile_one_output" and (p["waves"], p["rows"], p["sets"], p["outputs"]) == (4, rows, sets, 1)
        assert p["workgroups"] == 3 * 4096 // 64
    assert kaio.kaio_qkv_plan(129, 4096, 4096)["kernel"] == "tile"
    from tests.gpu_util import NO_INT8_FORMS, TILE_FORMS, form_of, shape_for_form
    for bits in (4, 8):
        for m, n, k in ((129, 4096, 4096), (777, 1000, 384), (2048, 4096, 4096), (5000, 12288, 4224),
                        (100, 1000, 384), (70, 4096, 4096)):
            p = kaio.kaio_qkv_plan(m, n, k, bits)
            assert p["kernel"] in ("tile", "tile_one_output") and form_of(p) in TILE_FORMS
            assert p["workgroups"] == -(-m // p["rows"]) * -(-n // (16 * p["waves"])) * (3 // p["outputs"])
            if p["sets"] > 1:   # the sets split the group count evenly; no INT8 form its rings do not fit
                assert (k // 128) % p["sets"] == 0 and not (bits == 8 and form_of(p) in NO_INT8_FORMS)
        # the prefill workload keeps the 8-wave 128-row form
        p = kaio.kaio_qkv_plan(2048, 4096, 4096, bits)
        assert form_of(p) == (8, 128, 1, 3)
        # every form the kernels have is chosen for some problem (INT8 lacks the forms whose rings
        # would not fit in LDS)
        for f in TILE_FORMS:
            found = shape_for_form(f, bits, True)
            assert (found is None) == (bits == 8 and f in NO_INT8_FORMS), (bits, f, found)
