// Internal launchers (host side).  The C ABI in kaio_abi.cpp validates every
// argument before calling these; the launchers assume valid, non-empty problems.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/kaio.h"

namespace kaio {

struct QkvProblem {
  const uint16_t* x;        // f16 [m, k]
  const uint32_t* w[3];     // u32 [k*bits/32, n]: INT4 (bits 4) or INT8 (bits 8) values packed along k
  const uint16_t* s[3];     // f16 [k/128, n]
  uint16_t* out[3];         // f16 [m, n]
  uint32_t m, n, k;
  uint32_t bits;            // 4 (W4A16) or 8 (W8A16)
};

// Tile geometry, shared with the host-side grid-size checks.
constexpr uint32_t kPrefillBM = 128;   // rows of x per workgroup
constexpr uint64_t kComputeUnits = 256;  // MI355X
// Waves per tile-kernel workgroup (each owns 16 columns of every output):
// 8, unless the grid of 4-wave workgroups (64 columns) still fits in one pass
// over the compute units -- then the narrower tiles double the workgroups.
constexpr int prefill_waves(uint32_t m, uint32_t n) {
  return (uint64_t)((m + kPrefillBM - 1) / kPrefillBM) * ((n + 63) / 64) <= kComputeUnits ? 4 : 8;
}
// columns of each output per tile-kernel workgroup
constexpr uint32_t prefill_bn(uint32_t m, uint32_t n) { return 16u * prefill_waves(m, n); }
// Rows per tile-kernel workgroup: 64 when a grid of 4-wave 64-row workgroups
// still fits one pass over the compute units (then the 128-row grid would
// leave many idle: 128 < m <= 256 at n = 4096), else 128.
constexpr uint32_t prefill_bm(uint32_t m, uint32_t n) {
  return (uint64_t)((m + 63) / 64) * ((n + 63) / 64) <= kComputeUnits ? 64u : kPrefillBM;
}
// 4-wave tiles run the groups as two halves on two sets of 4 waves when the
// group count is even (128-row tiles: INT4 only, whose two rings fit in LDS),
// else on one set
constexpr int prefill_ksplit(uint32_t m, uint32_t n, uint32_t k, uint32_t bits) {
  return prefill_waves(m, n) == 4 && (k / 128) % 2 == 0 && (prefill_bm(m, n) == 64 || bits == 4) ? 2 : 1;
}
constexpr uint32_t kMaxN = 1u << 26;   // keeps 32-bit per-lane byte offsets in range (16 rows x N x 4 B)
constexpr uint32_t kMaxK = 1u << 24;
#ifndef KAIO_SK_MAXM
#define KAIO_SK_MAXM 128
#endif
constexpr uint32_t kDecodeMaxM = KAIO_SK_MAXM;   // m <= this runs the split-K kernel
// split-K configuration for 32 < m <= 64: row tiles per wave (the other
// rows go to other waves), words per lane load, waves per workgroup
#ifndef KAIO_SK4_RT
#define KAIO_SK4_RT 2
#endif
#ifndef KAIO_SK4_VEC
#define KAIO_SK4_VEC 4
#endif
#ifndef KAIO_SK4_WAVES
#define KAIO_SK4_WAVES 8
#endif
// columns of one output per split-K workgroup, by row count
constexpr uint32_t decode_bn(uint32_t m) { return m <= 32 ? 64u : m <= 64 ? 16u * KAIO_SK4_VEC : 64u; }
// split-K configuration for 64 < m <= 128: row tiles per wave, waves per workgroup
#ifndef KAIO_SK8_RT
#define KAIO_SK8_RT 2
#endif
#ifndef KAIO_SK8_WAVES
#define KAIO_SK8_WAVES 8
#endif
constexpr uint32_t kGemmBM = 256;
constexpr uint32_t kGemmBN = 256;
constexpr uint64_t kMaxWorkgroups = (1ull << 24) - 1;  // 1-D grid limit at 256 threads

hipError_t launch_qkv_prefill(const QkvProblem& p, hipStream_t stream);
hipError_t launch_qkv_decode(const QkvProblem& p, hipStream_t stream);
hipError_t launch_fill_zero(void* dst, size_t bytes, hipStream_t stream);
// grad16 is caller-provided scratch for f16(grad), m * n halves.
hipError_t launch_gemm_f16f32_bwd(const uint16_t* a, const uint16_t* b, const float* grad, uint16_t* grad_a,
                                  uint16_t* grad_b, uint16_t* grad16, uint32_t m, uint32_t n, uint32_t k,
                                  hipStream_t stream);
// The same with f16(grad) in the library's static per-device buffer of
// kGemmBwdScratchBytes (m * n * 2 must fit); nothing is allocated.
constexpr uint64_t kGemmBwdScratchBytes = 64ull << 20;
hipError_t launch_gemm_f16f32_bwd_noalloc(const uint16_t* a, const uint16_t* b, const float* grad,
                                          uint16_t* grad_a, uint16_t* grad_b, uint32_t m, uint32_t n,
                                          uint32_t k, hipStream_t stream);
hipError_t launch_gemm_f16f32(const uint16_t* a, const uint16_t* b, float* c,
                              uint32_t m, uint32_t n, uint32_t k, hipStream_t stream);
hipError_t launch_dequant_group_bwd(kaio_dtype dtype, int64_t outer, int64_t axis,
                                    int64_t group, const void* dy, const void* scale,
                                    void* dq, hipStream_t stream);

}  // namespace kaio
