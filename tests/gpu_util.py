"""Helpers for the GPU parity tests (host <-> device copies only)."""
import numpy as np
import torch

DEV = torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32)).to(DEV)
    if a.dtype == np.uint16:                      # bf16 bit patterns
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def qkv_on_gpu(x, w, s, bits=4, **kw):
    import int4_group_quantized_w4a16_amd as kaio
    fn = kaio.kaio_qkv_w8a16 if bits == 8 else kaio.kaio_qkv_w4a16
    outs = fn(to_dev(x), *[to_dev(a) for a in w], *[to_dev(a) for a in s], **kw)
    torch.cuda.synchronize()
    return [to_host(o) for o in outs]
