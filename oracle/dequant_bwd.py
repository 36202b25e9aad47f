"""Per-group dequant straight-through backward -- oracle side (test infrastructure only).

Source: baracuda-kernels 0.0.1-alpha.68, src/quantize/dequantize_per_group_backward.rs
-- module doc (dq[i, j] = dy[i, j] * scale[i, j / group_size]),
``DequantizePerGroupBackwardArgs`` (d_output and d_input ``[outer, axis]``,
scale ``[outer, num_groups]``, all of one float dtype),
``DequantizePerGroupBackwardPlan::select`` (dtypes f32/f64/f16/bf16;
outer, axis >= 0; group > 0; axis a multiple of group) and ``run``
(an empty problem returns without work).

    dq[i, j] = round_T( dy[i, j] * scale[i, j // g] )

computed as an exact float64 product followed by one round-to-nearest-even
into the storage dtype T.  For f32, bf16 and f16 inputs the float64 product
is exact, so this is the correctly rounded product -- the single result a
"deterministic, bit-stable" multiply in T can give.  For f64 it is the
IEEE float64 multiply itself.
"""
from __future__ import annotations

import numpy as np

from .rounding import f64_to_storage, storage_to_f64

DTYPES = ("f32", "f64", "f16", "bf16")


def check_problem(outer: int, axis: int, group: int):
    if outer < 0 or axis < 0:
        raise ValueError("outer_size and axis_size must be non-negative")
    if group <= 0:
        raise ValueError("group_size must be > 0")
    if axis % group:
        raise ValueError("axis_size must be a multiple of group_size")


def dequant_bwd(dy, scale, group: int, dtype: str):
    """dy[outer, axis], scale[outer, axis/group] in storage dtype -> dq in storage dtype."""
    if dtype not in DTYPES:
        raise ValueError(f"unsupported dtype {dtype!r}")
    dy = np.asarray(dy)
    scale = np.asarray(scale)
    outer, axis = dy.shape
    check_problem(outer, axis, group)
    if scale.shape != (outer, axis // group):
        raise ValueError("scale shape != [outer, num_groups]")
    dy64 = storage_to_f64(dy, dtype)
    sc64 = storage_to_f64(scale, dtype)
    group_of_j = np.arange(axis) // group
    return f64_to_storage(dy64 * sc64[:, group_of_j], dtype)
