"""Seeded synthetic workloads shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and casts them to their storage dtypes
(numpy / torch casts, round-to-nearest-even).  It contains none of the
arithmetic of the operations themselves: no nibble decoding, no scaling, no
products or sums.  Both the CPU oracle and the GPU library consume the exact
bytes produced here.

Packed INT4 weights are drawn as uniform random ``uint32`` words.  Every one of
the 2**32 words is a distinct packing of eight 4-bit fields, so a uniform word
is the same thing as eight independent nibbles, each uniform over its 16
values -- i.e. eight independent signed INT4 values uniform in [-8, 7] under
the two's-complement reading.  No packing code is needed to produce them.

Shapes and distributions follow the workload table of the pages' three
operations (kaio-candle ``qkv_project_int4``, kaio-candle ``matmul_tc_async``,
baracuda-kernels ``dequantize_per_group_backward``):

* QKV:  x f16[M,K] ~ N(0,1); 3 x u32[K/8,N] uniform words; 3 x f16[K/128,N]
  ~ U[0.005, 0.02].  Draw order: x, w_q, w_k, w_v, s_q, s_k, s_v.
* W8A16 QKV (the INT8 sibling): x f16[M,K] ~ N(0,1); 3 x u32[K/4,N] uniform
  words (four independent INT8 values uniform in [-128, 127] each, by the same
  argument as for INT4); 3 x f16[K/128,N] ~ U[0.0003125, 0.00125] -- the INT4
  scale range divided by 16, so that the dequantized weights span the same
  range as the INT4 workload's.  Draw order: x, w_q, w_k, w_v, s_q, s_k, s_v.
* GEMM: A f16[M,K], B f16[K,N] ~ N(0,1).  Draw order: A, B.
* Dequant backward: dy[outer,axis] ~ N(0,1), scale[outer,axis/g] ~ U[0.001, 0.1],
  drawn in f64, cast to the storage dtype.  Draw order: dy, scale.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

GROUP = 128

# Named workloads (sizes and seeds).
QKV_TINY = dict(M=16, N=512, K=512, seed=1001)
GEMM_4096 = dict(M=4096, N=4096, K=4096, seed=1002, check_seed=1012)
QKV_DECODE = dict(M=8, N=4096, K=4096, seed=1003, rotate=21)
QKV_PREFILL = dict(M=2048, N=4096, K=4096, seed=1004)
DEQUANT_BWD = dict(outer=16384, axis=8192, group=128, seed=1005)
# W8A16 sibling at the INT4 workloads' shapes
QKV8_TINY = dict(M=16, N=512, K=512, seed=1101)
QKV8_DECODE = dict(M=8, N=4096, K=4096, seed=1103, rotate=11)
QKV8_PREFILL = dict(M=2048, N=4096, K=4096, seed=1104)
QKV8_SCALE_LO, QKV8_SCALE_HI = 0.005 / 16, 0.02 / 16


@dataclass
class QKVInputs:
    x: np.ndarray            # f16 [M, K]
    w: tuple                 # 3 x u32 [K/8, N]  (q, k, v)
    s: tuple                 # 3 x f16 [K/128, N] (q, k, v)

    @property
    def shape(self):
        M, K = self.x.shape
        return M, self.w[0].shape[1], K


def qkv_inputs(M: int, N: int, K: int, seed: int,
               scale_lo: float = 0.005, scale_hi: float = 0.02) -> QKVInputs:
    if K % 8:
        raise ValueError("K must be a multiple of 8 to form packed rows")
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float16)
    w = tuple(rng.integers(0, 2 ** 32, size=(K // 8, N), dtype=np.uint32) for _ in range(3))
    g = K // GROUP
    s = tuple(rng.uniform(scale_lo, scale_hi, size=(g, N)).astype(np.float16) for _ in range(3))
    return QKVInputs(x=x, w=w, s=s)


def qkv8_inputs(M: int, N: int, K: int, seed: int,
                scale_lo: float = QKV8_SCALE_LO, scale_hi: float = QKV8_SCALE_HI) -> QKVInputs:
    """W8A16 inputs: packed weights u32[K/4, N] (four INT8 values per word)."""
    if K % 4:
        raise ValueError("K must be a multiple of 4 to form packed rows")
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float16)
    w = tuple(rng.integers(0, 2 ** 32, size=(K // 4, N), dtype=np.uint32) for _ in range(3))
    g = K // GROUP
    s = tuple(rng.uniform(scale_lo, scale_hi, size=(g, N)).astype(np.float16) for _ in range(3))
    return QKVInputs(x=x, w=w, s=s)


def qkv8_weight_set(N: int, K: int, seed: int,
                    scale_lo: float = QKV8_SCALE_LO, scale_hi: float = QKV8_SCALE_HI):
    """A fresh W8A16 (w_q, w_k, w_v, s_q, s_k, s_v) set, used to rotate decode weights."""
    rng = np.random.default_rng(seed)
    w = tuple(rng.integers(0, 2 ** 32, size=(K // 4, N), dtype=np.uint32) for _ in range(3))
    s = tuple(rng.uniform(scale_lo, scale_hi, size=(K // GROUP, N)).astype(np.float16)
              for _ in range(3))
    return w, s


def qkv_weight_set(N: int, K: int, seed: int,
                   scale_lo: float = 0.005, scale_hi: float = 0.02):
    """A fresh (w_q, w_k, w_v, s_q, s_k, s_v) set, used to rotate decode weights."""
    rng = np.random.default_rng(seed)
    w = tuple(rng.integers(0, 2 ** 32, size=(K // 8, N), dtype=np.uint32) for _ in range(3))
    s = tuple(rng.uniform(scale_lo, scale_hi, size=(K // GROUP, N)).astype(np.float16)
              for _ in range(3))
    return w, s


def gemm_inputs(M: int, N: int, K: int, seed: int):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((M, K)).astype(np.float16)
    b = rng.standard_normal((K, N)).astype(np.float16)
    return a, b


def gemm_check_positions(M: int, N: int, count: int, seed: int, block: int = 256):
    """Positions checked at full GEMM size: a leading block plus seeded random entries."""
    rng = np.random.default_rng(seed)
    bi, bj = np.meshgrid(np.arange(min(block, M)), np.arange(min(block, N)), indexing="ij")
    ri = rng.integers(0, M, size=count)
    rj = rng.integers(0, N, size=count)
    return (np.concatenate([bi.ravel(), ri]).astype(np.int64),
            np.concatenate([bj.ravel(), rj]).astype(np.int64))


def _to_bf16_bits(a64: np.ndarray) -> np.ndarray:
    """Cast through torch (f64 -> f32 -> bf16, both casts RNE); returns uint16 bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a64, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def dequant_bwd_inputs(outer: int, axis: int, group: int, seed: int, dtype: str):
    """dy[outer, axis], scale[outer, axis/group] in the storage dtype.

    ``dtype`` is one of "f32", "bf16", "f16", "f64".  bf16 arrays are returned as
    uint16 bit patterns (numpy has no bfloat16).
    """
    if group <= 0 or axis % group:
        raise ValueError("axis must be a positive multiple of group")
    rng = np.random.default_rng(seed)
    dy = rng.standard_normal((outer, axis))
    sc = rng.uniform(0.001, 0.1, size=(outer, axis // group))
    if dtype == "f32":
        return dy.astype(np.float32), sc.astype(np.float32)
    if dtype == "f64":
        return dy, sc
    if dtype == "f16":
        return dy.astype(np.float16), sc.astype(np.float16)
    if dtype == "bf16":
        return _to_bf16_bits(dy), _to_bf16_bits(sc)
    raise ValueError(f"unknown dtype {dtype!r}")
