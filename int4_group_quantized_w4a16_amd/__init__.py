"""MI355X (gfx950) W4A16 fused-QKV library (and its W8A16 sibling): thin Python binding over libkaio.so.

Every function here only marshals arguments (shape/dtype/device checks,
output allocation through PyTorch, the current HIP stream) and calls the
C ABI declared in ``include/kaio.h``.  All arithmetic runs in the HIP
kernels; there is no CPU fallback -- if ``libkaio.so`` is missing or the
device is not gfx950 the call raises.

    kaio_qkv_w4a16(x, w_q, w_k, w_v, s_q, s_k, s_v) -> (q, k, v)
    kaio_qkv_w8a16(x, w_q, w_k, w_v, s_q, s_k, s_v) -> (q, k, v)
    kaio_gemm_f16f32(a, b) -> c
    kaio_gemm_f16f32_bwd(a, b, grad) -> (grad_a, grad_b)
    kaio_dequant_group_bwd(dy, scale, group_size) -> dq
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["DTYPE_CODES", "KaioError", "kaio_qkv_w4a16", "kaio_qkv_w8a16", "kaio_gemm_f16f32", "kaio_gemm_f16f32_bwd",
           "kaio_dequant_group_bwd",
           "kaio_last_error", "kaio_version", "lib", "LIB_PATH", "GROUP_SIZE"]

# KAIO_LIBRARY may name another in-tree build of the same library (the host-sanitizer
# build used by the CPU boundary tests); by default the in-tree libkaio.so is loaded.
LIB_PATH = os.environ.get("KAIO_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkaio.so")
GROUP_SIZE = 128

STATUS = {0: "OK", 1: "INVALID_ARGUMENT", 2: "INVALID_PROBLEM", 3: "UNSUPPORTED", 4: "DEVICE", 5: "LAUNCH"}
DTYPE_CODES = {"f32": 0, "bf16": 1, "f16": 2, "f64": 3}


class KaioError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{STATUS.get(status, status)}] {message}")
        self.status = status
        self.message = message


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C library (loads on first use; raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m int4_group_quantized_w4a16_amd.build_lib`")
        L = ctypes.CDLL(LIB_PATH)
        vp, u32, i32 = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_int32
        L.kaio_qkv_w4a16.argtypes = [vp] * 10 + [u32] * 4 + [vp]
        L.kaio_qkv_w4a16.restype = ctypes.c_int
        L.kaio_qkv_w8a16.argtypes = [vp] * 10 + [u32] * 4 + [vp]
        L.kaio_qkv_w8a16.restype = ctypes.c_int
        L.kaio_gemm_f16f32.argtypes = [vp, vp, vp, u32, u32, u32, vp]
        L.kaio_gemm_f16f32.restype = ctypes.c_int
        L.kaio_gemm_f16f32_bwd.argtypes = [vp] * 5 + [u32] * 3 + [vp, ctypes.c_size_t, vp]
        L.kaio_gemm_f16f32_bwd.restype = ctypes.c_int
        L.kaio_gemm_f16f32_bwd_noalloc.argtypes = [vp] * 5 + [u32] * 3 + [vp]
        L.kaio_gemm_f16f32_bwd_noalloc.restype = ctypes.c_int
        L.kaio_gemm_f16f32_bwd_workspace_size.argtypes = [u32, u32]
        L.kaio_gemm_f16f32_bwd_workspace_size.restype = ctypes.c_size_t
        L.kaio_dequant_group_bwd.argtypes = [ctypes.c_int, i32, i32, i32, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.kaio_dequant_group_bwd.restype = ctypes.c_int
        L.kaio_qkv_plan.argtypes = [u32] * 4 + [vp]
        L.kaio_qkv_plan.restype = ctypes.c_int
        L.kaio_last_error.argtypes = []
        L.kaio_last_error.restype = ctypes.c_char_p
        L.kaio_version.argtypes = []
        L.kaio_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def kaio_last_error() -> str:
    return lib().kaio_last_error().decode()


def kaio_version() -> str:
    return lib().kaio_version().decode()


def kaio_qkv_plan(m: int, n: int, k: int, bits: int = 4) -> dict:
    """The kernel form a QKV call of these sizes runs (kaio_qkv_plan; host only)."""
    plan = (ctypes.c_uint32 * 5)()
    _check(lib().kaio_qkv_plan(m, n, k, bits, plan))
    return {"kernel": ("split_k", "tile", "tile_one_output")[plan[0]], "waves": plan[1], "rows": plan[2],
            "sets": plan[3], "outputs": 1 if plan[0] == 2 else 3, "workgroups": plan[4]}


def _check(status: int):
    if status != 0:
        raise KaioError(status, kaio_last_error())


def _stream(device, stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _tensor(t, name, dtypes, device=None, rank=2):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dim() != rank:
        raise ValueError(f"{name} must be rank-{rank}, got shape {tuple(t.shape)}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device; there is no CPU fallback")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous() or t.storage_offset() != 0:
        raise ValueError(f"{name} must be contiguous with zero offset")
    return t


def _u32_dtypes():
    import torch
    return (torch.int32, torch.uint32) if hasattr(torch, "uint32") else (torch.int32,)


def _qkv(fn, bits, x, w_q, w_k, w_v, s_q, s_k, s_v, q, k, v, stream):
    import torch
    f16 = (torch.float16,)
    _tensor(x, "x", f16)
    dev = x.device
    M, K = x.shape
    per_word = 32 // bits
    ws = [_tensor(t, n, _u32_dtypes(), dev) for t, n in ((w_q, "w_q_packed"), (w_k, "w_k_packed"), (w_v, "w_v_packed"))]
    ss = [_tensor(t, n, f16, dev) for t, n in ((s_q, "scales_q"), (s_k, "scales_k"), (s_v, "scales_v"))]
    if K % GROUP_SIZE:
        raise ValueError(f"K ({K}) must be a multiple of group_size ({GROUP_SIZE})")
    for t, n in zip(ws, ("w_q_packed", "w_k_packed", "w_v_packed")):
        if t.shape[0] != K // per_word:
            raise ValueError(f"{n} has {t.shape[0]} rows, expected K/{per_word} = {K // per_word} (K={K})")
    for t, n in zip(ss, ("scales_q", "scales_k", "scales_v")):
        if t.shape[0] != K // GROUP_SIZE:
            raise ValueError(f"{n} has {t.shape[0]} rows, expected K/{GROUP_SIZE} = {K // GROUP_SIZE} (K={K})")
    Ns = [t.shape[1] for t in ws + ss]
    if len(set(Ns)) != 1:
        raise ValueError(f"N mismatch across weight/scale tensors: {Ns}")
    N = Ns[0]
    outs = []
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if t is None:
            t = torch.empty((M, N), dtype=torch.float16, device=dev)
        _tensor(t, n, f16, dev)
        if tuple(t.shape) != (M, N):
            raise ValueError(f"output {n} must be [{M}, {N}]")
        outs.append(t)
    for dim in (M, N, K):
        if dim >= 2 ** 32:
            raise ValueError("dimension exceeds u32")
    _check(fn(x.data_ptr(), *[t.data_ptr() for t in ws], *[t.data_ptr() for t in ss],
              *[t.data_ptr() for t in outs], M, N, K, GROUP_SIZE, _stream(dev, stream)))
    return tuple(outs)


def kaio_qkv_w4a16(x, w_q, w_k, w_v, s_q, s_k, s_v, q=None, k=None, v=None, stream=None):
    """Fused W4A16 QKV projection; returns (q, k, v), each f16[M, N].

    x f16[M,K]; w_* packed INT4 as int32/uint32 [K/8, N]; s_* f16[K/128, N].
    """
    return _qkv(lib().kaio_qkv_w4a16, 4, x, w_q, w_k, w_v, s_q, s_k, s_v, q, k, v, stream)


def kaio_qkv_w8a16(x, w_q, w_k, w_v, s_q, s_k, s_v, q=None, k=None, v=None, stream=None):
    """Fused W8A16 QKV projection; returns (q, k, v), each f16[M, N].

    x f16[M,K]; w_* packed INT8 as int32/uint32 [K/4, N] (byte i of row r holds k = 4r+i);
    s_* f16[K/128, N].
    """
    return _qkv(lib().kaio_qkv_w8a16, 8, x, w_q, w_k, w_v, s_q, s_k, s_v, q, k, v, stream)


def kaio_gemm_f16f32(a, b, c=None, stream=None):
    """C = A . B with A f16[M,K], B f16[K,N]; returns C f32[M,N]."""
    import torch
    _tensor(a, "a", (torch.float16,))
    _tensor(b, "b", (torch.float16,), a.device)
    M, K = a.shape
    Kb, N = b.shape
    if K != Kb:
        raise ValueError(f"K mismatch between inputs: a is [{M}, {K}], b is [{Kb}, {N}]")
    if c is None:
        c = torch.empty((M, N), dtype=torch.float32, device=a.device)
    _tensor(c, "c", (torch.float32,), a.device)
    if tuple(c.shape) != (M, N):
        raise ValueError(f"c must be [{M}, {N}]")
    _check(lib().kaio_gemm_f16f32(a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, K, _stream(a.device, stream)))
    return c


def kaio_gemm_f16f32_bwd(a, b, grad, grad_a=None, grad_b=None, workspace=None, stream=None):
    """Backward of C = A . B: returns (grad_a f16[M,K], grad_b f16[K,N]) for grad f32[M,N].

    grad is cast to f16 first; each gradient is accumulated in f32 and rounded to f16.
    ``workspace`` (uint8, at least M*N*2 bytes) is allocated here when not given.
    """
    import torch
    _tensor(a, "a", (torch.float16,))
    _tensor(b, "b", (torch.float16,), a.device)
    _tensor(grad, "grad", (torch.float32,), a.device)
    M, K = a.shape
    Kb, N = b.shape
    if K != Kb or tuple(grad.shape) != (M, N):
        raise ValueError(f"shape mismatch: a [{M}, {K}], b [{Kb}, {N}], grad {list(grad.shape)}")
    if grad_a is None:
        grad_a = torch.empty((M, K), dtype=torch.float16, device=a.device)
    if grad_b is None:
        grad_b = torch.empty((K, N), dtype=torch.float16, device=a.device)
    _tensor(grad_a, "grad_a", (torch.float16,), a.device)
    _tensor(grad_b, "grad_b", (torch.float16,), a.device)
    if tuple(grad_a.shape) != (M, K) or tuple(grad_b.shape) != (K, N):
        raise ValueError(f"grad_a must be [{M}, {K}] and grad_b [{K}, {N}]")
    need = lib().kaio_gemm_f16f32_bwd_workspace_size(M, N)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=a.device)
    _tensor(workspace, "workspace", (torch.uint8,), a.device, rank=1)
    _check(lib().kaio_gemm_f16f32_bwd(a.data_ptr(), b.data_ptr(), grad.data_ptr(), grad_a.data_ptr(),
                                      grad_b.data_ptr(), M, N, K, workspace.data_ptr(), workspace.numel(),
                                      _stream(a.device, stream)))
    return grad_a, grad_b


def kaio_dequant_group_bwd(dy, scale, group_size, dq=None, stream=None):
    """dq[i, j] = dy[i, j] * scale[i, j // group_size], bit-exact, same dtype as dy."""
    import torch
    codes = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2, torch.float64: 3}
    _tensor(dy, "d_output", tuple(codes))
    _tensor(scale, "scale", (dy.dtype,), dy.device)
    outer, axis = dy.shape
    if group_size <= 0 or axis % group_size:
        raise ValueError("axis_size must be a positive multiple of group_size")
    if tuple(scale.shape) != (outer, axis // group_size):
        raise ValueError("scale shape != [outer, num_groups]")
    if dq is None:
        dq = torch.empty_like(dy)
    _tensor(dq, "d_input", (dy.dtype,), dy.device)
    if tuple(dq.shape) != (outer, axis):
        raise ValueError("d_input shape != [outer, axis_size]")
    if outer >= 2 ** 31 or axis >= 2 ** 31:
        raise ValueError("sizes exceed i32")
    _check(lib().kaio_dequant_group_bwd(codes[dy.dtype], outer, axis, group_size, dy.data_ptr(),
                                        scale.data_ptr(), dq.data_ptr(), None, 0, _stream(dy.device, stream)))
    return dq
