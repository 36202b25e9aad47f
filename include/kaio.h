/*
 * kaio.h -- C ABI of the MI355X (gfx950) W4A16 fused-QKV library.
 *
 * Each operation is one asynchronous launch on the caller's HIP stream:
 *
 *   kaio_qkv_w4a16          W4A16 group-quantized fused tri-output QKV projection
 *   kaio_qkv_w8a16          its W8A16 sibling (INT8 weights, same contract)
 *                           (kaio_qkv_plan: which kernel form a call of given sizes runs)
 *   kaio_gemm_f16f32        dense f16 x f16 -> f32 matmul
 *   kaio_gemm_f16f32_bwd    its backward: f16 gradients of A and B
 *                           (kaio_gemm_f16f32_bwd_noalloc: the same without a workspace)
 *   kaio_dequant_group_bwd  straight-through per-group dequant backward
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 * - Pointers are DEVICE pointers (memory the HIP runtime allocated on the
 *   current device).  The caller owns every buffer; the library never
 *   allocates, frees, copies to the host or synchronizes.  Inputs are never
 *   written.  Outputs are fully overwritten (no pre-zeroing needed).
 * - All tensors are dense, row-major, zero-offset.  Base pointers must be
 *   16-byte aligned.  Outputs must not overlap any input or each other.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).  The
 *   launch is queued on it and the call returns; a fault inside a kernel is
 *   reported by the caller's next synchronizing HIP call, not here.
 * - Validation happens on the host, in the order listed per entry point;
 *   the first failure wins and nothing is launched.  An empty problem
 *   (no outputs) returns KAIO_OK without touching the device.
 * - On failure kaio_last_error() returns "kaio::<op>: <reason>" for the
 *   calling thread.
 * - The device must be an AMD gfx950 (MI355X); anything else returns
 *   KAIO_ERR_DEVICE.  There is no CPU fallback.
 */
#ifndef KAIO_H
#define KAIO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kaio_status {
  KAIO_OK = 0,
  KAIO_ERR_INVALID_ARGUMENT = 1, /* null, misaligned or overlapping pointer             */
  KAIO_ERR_INVALID_PROBLEM = 2,  /* sizes the operation does not define                 */
  KAIO_ERR_UNSUPPORTED = 3,      /* defined, but not offered (group size, dtype)        */
  KAIO_ERR_DEVICE = 4,           /* no HIP device, or the current device is not gfx950 */
  KAIO_ERR_LAUNCH = 5            /* the HIP runtime refused the launch                  */
} kaio_status;

typedef enum kaio_dtype {
  KAIO_DTYPE_F32 = 0,
  KAIO_DTYPE_BF16 = 1,
  KAIO_DTYPE_F16 = 2,
  KAIO_DTYPE_F64 = 3
} kaio_dtype;

/*
 * W4A16 fused tri-output QKV projection.
 * Defined by: kaio-candle 0.2.0, src/qkv_project_int4.rs -- module doc (one
 * launch, seven inputs, group size locked at 128, K a multiple of 128) and
 * the doc comment of qkv_project_int4 (operand shapes, f16 outputs converted
 * from f32 inside the kernel).
 *
 *   For p in {q, k, v}:
 *     Y_p[m, n] = sum_k x[m, k] * int4(W_p, k, n) * S_p[k / 128, n]
 *
 *   x        f16[m, k]       activations, shared by the three projections
 *   w_q/k/v  u32[k/8, n]     packed INT4 weights: word (r, n) at offset r*n_cols + n;
 *                            nibble i (bits 4i..4i+3, low first) holds k = 8r + i as a
 *                            signed two's-complement value in [-8, 7], no zero point
 *   s_q/k/v  f16[k/128, n]   one scale per 128 consecutive k of each column
 *   q, k_out, v  f16[m, n]   outputs, f32 accumulation rounded once to f16 (RNE)
 *   group_size  must be 128
 *
 * Validation order: group_size != 128 -> UNSUPPORTED; k % 128 != 0 ->
 * INVALID_PROBLEM; m == 0 or n == 0 -> OK (nothing launched); sizes too
 * large for one launch (n >= 2^26, k >= 2^24, any tensor of 2^62 bytes or
 * more, or more than 2^24 - 1 workgroups) -> INVALID_PROBLEM; null pointer (weights/scales/x
 * only when k > 0) -> INVALID_ARGUMENT; misaligned pointer ->
 * INVALID_ARGUMENT; an output overlapping an input or another output ->
 * INVALID_ARGUMENT; device -> DEVICE; launch -> LAUNCH.  k == 0 writes
 * zeros.  m <= 64 runs the memory-bound split-K kernel (decode and batched
 * decode), larger m the MFMA tile kernel (up to m = 128 with one output per
 * workgroup, and so from m = 33 when k / 128 is a multiple of 4); all obey
 * this contract.
 */
kaio_status kaio_qkv_w4a16(const void* x,
                           const uint32_t* w_q, const uint32_t* w_k, const uint32_t* w_v,
                           const void* s_q, const void* s_k, const void* s_v,
                           void* q, void* k_out, void* v,
                           uint32_t m, uint32_t n, uint32_t k, uint32_t group_size,
                           void* stream);

/*
 * W8A16 fused tri-output QKV projection: the INT8 sibling of kaio_qkv_w4a16.
 * Named by: kaio-candle 0.2.0, src/qkv_project_int4.rs -- module doc (the
 * INT4 op follows the same direct-call pattern as qkv_project_int8, whose
 * weight layout the pages do not print).  This library's reading of it is the
 * 8-bit analogue of the INT4 packing:
 *
 *   For p in {q, k, v}:
 *     Y_p[m, n] = sum_k x[m, k] * int8(W_p, k, n) * S_p[k / 128, n]
 *
 *   x        f16[m, k]       activations, shared by the three projections
 *   w_q/k/v  u32[k/4, n]     packed INT8 weights: word (r, n) at offset r*n_cols + n;
 *                            byte i (bits 8i..8i+7, low first) holds k = 4r + i as a
 *                            signed two's-complement value in [-128, 127], no zero point
 *   s_q/k/v  f16[k/128, n]   one scale per 128 consecutive k of each column
 *   q, k_out, v  f16[m, n]   outputs, f32 accumulation rounded once to f16 (RNE)
 *   group_size  must be 128
 *
 * Validation order, limits and error behaviour: exactly as kaio_qkv_w4a16;
 * m <= 64 runs the split-K kernel, larger m the tile kernel.
 */
kaio_status kaio_qkv_w8a16(const void* x,
                           const uint32_t* w_q, const uint32_t* w_k, const uint32_t* w_v,
                           const void* s_q, const void* s_k, const void* s_v,
                           void* q, void* k_out, void* v,
                           uint32_t m, uint32_t n, uint32_t k, uint32_t group_size,
                           void* stream);

/*
 * Dense f16 x f16 -> f32 matmul, C = A . B (C is overwritten, not accumulated).
 * Defined by: kaio-candle 0.2.0, src/matmul_tc_async.rs -- module doc
 * (f16 x f16 -> f32 matmul) and MatmulTcAsyncOp::cuda_fwd (A [m, k],
 * B [k, n], a zeroed [m, n] f32 output written by the kernel).
 *
 *   a  f16[m, k]   b  f16[k, n]   c  f32[m, n]
 *
 * Validation order: m == 0 or n == 0 -> OK (nothing launched); sizes too
 * large for one launch -> INVALID_PROBLEM; null pointer (a, b only when
 * k > 0) -> INVALID_ARGUMENT; misaligned -> INVALID_ARGUMENT; c overlapping
 * a or b -> INVALID_ARGUMENT; device -> DEVICE; launch -> LAUNCH.  k == 0
 * writes zeros.
 */
kaio_status kaio_gemm_f16f32(const void* a, const void* b, float* c,
                             uint32_t m, uint32_t n, uint32_t k, void* stream);

/*
 * Backward of kaio_gemm_f16f32 for an f32 output gradient g [m, n]:
 *   g16    = f16(g)                                (round to nearest even)
 *   grad_a = f16( g16 . b^T )     f16[m, k]
 *   grad_b = f16( a^T . g16 )     f16[k, n]
 * each product accumulated in f32 and rounded once to f16 (nearest even).
 * Defined by: kaio-candle 0.2.0, src/matmul_tc_async.rs --
 * MatmulTcAsyncOp::bwd (the gradient cast to f16, dA = grad . B^T and
 * dB = A^T . grad by the forward kernel, both results cast to f16).
 *
 *   a  f16[m, k]   b  f16[k, n]   grad  f32[m, n]
 *   grad_a  f16[m, k]   grad_b  f16[k, n]
 *   workspace  device scratch for g16: at least
 *              kaio_gemm_f16f32_bwd_workspace_size(m, n) bytes, 16-byte
 *              aligned, overlapping nothing else; its contents on return
 *              are unspecified.  Calls on one workspace must not overlap.
 *
 * Validation order: sizes too large for one launch -> INVALID_PROBLEM;
 * k == 0 -> OK (both gradients are empty, nothing launched); null output
 * -> INVALID_ARGUMENT; m == 0 or n == 0 -> both gradients are the empty
 * sum: zeros are written (a, b, grad and workspace are not read and may be
 * null); null input or workspace, or workspace_bytes too small ->
 * INVALID_ARGUMENT; misaligned -> INVALID_ARGUMENT; overlapping buffers ->
 * INVALID_ARGUMENT; device -> DEVICE; launch -> LAUNCH.
 */
kaio_status kaio_gemm_f16f32_bwd(const void* a, const void* b, const float* grad,
                                 void* grad_a, void* grad_b,
                                 uint32_t m, uint32_t n, uint32_t k,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes kaio_gemm_f16f32_bwd needs for an [m, n] gradient: m * n * 2. */
size_t kaio_gemm_f16f32_bwd_workspace_size(uint32_t m, uint32_t n);

/*
 * kaio_gemm_f16f32_bwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  f16(grad) is staged in a static device
 * buffer of KAIO_GEMM_BWD_NOALLOC_MAX_BYTES bytes that the library's code
 * object holds on every device it is loaded on, until the process ends; this
 * call allocates and frees nothing.  Results are bit-identical to
 * kaio_gemm_f16f32_bwd with a caller workspace (same kernels).
 *
 * Every call on a device shares that device's buffer: calls that overlap in
 * time on one device (other streams, concurrently replayed graphs) race and
 * must be serialized by the caller.  Nothing in the buffer needs to be
 * cleared between calls (the cast overwrites what the products read).
 *
 * Validation order: as kaio_gemm_f16f32_bwd, without the workspace checks,
 * plus m * n * 2 > KAIO_GEMM_BWD_NOALLOC_MAX_BYTES -> UNSUPPORTED (right
 * after the size check; nothing launched).
 */
#define KAIO_GEMM_BWD_NOALLOC_MAX_BYTES (64ull << 20)
kaio_status kaio_gemm_f16f32_bwd_noalloc(const void* a, const void* b, const float* grad,
                                         void* grad_a, void* grad_b,
                                         uint32_t m, uint32_t n, uint32_t k, void* stream);

/*
 * Straight-through per-group dequant backward:
 *   dq[i, j] = dy[i, j] * scale[i, j / group_size]     (one rounded multiply)
 * Defined by: baracuda-kernels 0.0.1-alpha.68,
 * src/quantize/dequantize_per_group_backward.rs -- module doc (the formula),
 * DequantizePerGroupBackwardArgs (shapes), DequantizePerGroupBackwardPlan::select
 * (dtype and size rules), ::workspace_size (none) and ::run (empty problem
 * returns without work).  Results are bit-exact: the correctly rounded
 * product in the dtype, identical on every run.
 *
 *   dtype      element type of dy, scale and dq (F32, BF16, F16, F64)
 *   dy         [outer, axis]              upstream gradient
 *   scale      [outer, axis / group_size] saved scales
 *   dq         [outer, axis]              output gradient
 *   workspace, workspace_bytes   accepted and ignored (no workspace is used)
 *
 * Pointers need only element alignment here; 16-byte alignment and
 * group_size % (16 / element size) == 0 select the vector path.
 *
 * Validation order: dtype unknown -> UNSUPPORTED; outer < 0 or axis < 0 ->
 * INVALID_PROBLEM; group_size <= 0 -> INVALID_PROBLEM; axis % group_size != 0
 * -> INVALID_PROBLEM; outer * axis == 0 -> OK (nothing launched); sizes
 * too large -> INVALID_PROBLEM; null pointer -> INVALID_ARGUMENT; misaligned (element) -> INVALID_ARGUMENT;
 * dq overlapping dy or scale -> INVALID_ARGUMENT; device -> DEVICE; launch
 * -> LAUNCH.
 */
kaio_status kaio_dequant_group_bwd(kaio_dtype dtype, int32_t outer, int32_t axis,
                                   int32_t group_size,
                                   const void* dy, const void* scale, void* dq,
                                   void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * Which kernel form a kaio_qkv_w4a16 (bits 4) or kaio_qkv_w8a16 (bits 8)
 * call of these sizes runs, for tests and tuning; host only, no device
 * touched, nothing launched.  On KAIO_OK:
 *   plan[0]  0: the split-K kernel, 1: the tile kernel (each workgroup
 *            computes its tile of Q, K and V), 2: the tile kernel with one
 *            output per workgroup (three times the workgroups)
 *   plan[1]  tile kernel: waves per set; split-K: 0
 *   plan[2]  tile kernel: rows of x per tile; split-K: columns per strip
 *   plan[3]  tile kernel: sets of waves per workgroup (2: the 128-k groups
 *            are split in halves over two sets); split-K: 1
 *   plan[4]  workgroups the launch has
 * m == 0 or n == 0 is an empty call (plan[0..4] = 0).  bits other than 4 or
 * 8, or a null plan -> INVALID_ARGUMENT; k % 128 != 0 -> INVALID_PROBLEM.
 */
kaio_status kaio_qkv_plan(uint32_t m, uint32_t n, uint32_t k, uint32_t bits, uint32_t plan[5]);

/* Message of the calling thread's most recent failed call ("" after a success). */
const char* kaio_last_error(void);

/* Library version string, e.g. "kaio-mi355x 0.1.0 gfx950". */
const char* kaio_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KAIO_H */
