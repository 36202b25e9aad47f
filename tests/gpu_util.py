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


# Forms of the tile kernel as kaio_qkv_plan reports them: (waves per set, rows per tile, sets of
# waves, outputs per workgroup)
TILE_FORMS = [(8, 128, 1, 3), (8, 96, 1, 3), (4, 128, 2, 3), (4, 96, 2, 3), (4, 64, 2, 3), (4, 128, 1, 3),
              (4, 96, 1, 3), (4, 64, 1, 3), (4, 128, 2, 1), (4, 96, 2, 1), (4, 128, 1, 1), (4, 96, 1, 1),
              (4, 64, 4, 1)]
# forms the INT8 kernels do not have (their rings would not fit in LDS)
NO_INT8_FORMS = [(4, 128, 2, 3), (4, 64, 4, 1)]


def form_of(plan):
    return (plan["waves"], plan["rows"], plan["sets"], plan["outputs"])


def shape_for_form(form, bits, aligned, ks=(256, 384, 512, 640)):
    """The smallest problem (m * n * k) of a coarse grid -- m ragged against every tile height,
    n % 8 == 0 or not -- on which the library's plan runs the tile kernel in `form`; None if
    no problem of the grid does."""
    import int4_group_quantized_w4a16_amd as kaio
    best = None
    for k in ks:
        for j in range(1, 33):
            n = 64 * j if aligned else 64 * j - 3
            for m in range(33, 2601, 13):
                if best is not None and m * n * k >= best[0]:
                    break
                p = kaio.kaio_qkv_plan(m, n, k, bits)
                if p["kernel"] != "split_k" and form_of(p) == tuple(form):
                    best = (m * n * k, m, n, k)
                    break
    return None if best is None else best[1:]
