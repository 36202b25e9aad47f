"""CPU oracle for the W4A16 fused-QKV library -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct float64 implementations of what the three
operations compute, written from the pages that define them:

* ``qkv``          -- the W4A16 group-quantized fused tri-output QKV projection
                      (kaio-candle 0.2.0, src/qkv_project_int4.rs, module doc and
                      the doc comment of ``qkv_project_int4``), and with ``bits=8``
                      its W8A16 sibling named in that module doc.
* ``gemm``         -- the dense f16 x f16 -> f32 matmul
                      (kaio-candle 0.2.0, src/matmul_tc_async.rs, module doc).
* ``gemm_bwd``     -- its backward: f16 gradients of A and B from an f32 output
                      gradient (same file, ``MatmulTcAsyncOp::bwd``).
* ``dequant_bwd``  -- the straight-through per-group dequant backward
                      (baracuda-kernels 0.0.1-alpha.68,
                      src/quantize/dequantize_per_group_backward.rs, module doc).
* ``int4``, ``int8``, ``rounding``, ``compare`` -- nibble and byte decoding,
                      IEEE rounding to a narrow format, and the parity tolerances.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never imports, links or
calls it, and this package shares no code with the GPU library: its nibble
decoder, rounding and accumulation are written independently.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against hand-worked cases (``tests/golden/``), exact rational brute force,
closed forms, or a library routine it does not itself call.
"""
from . import int4, int8, rounding, qkv, gemm, gemm_bwd, dequant_bwd, compare  # noqa: F401
