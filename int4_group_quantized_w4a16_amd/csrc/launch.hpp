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
constexpr uint64_t kComputeUnits = 256;  // MI355X
// Forms of the tile kernel: waves per set (each wave owns 16 columns of every
// output it computes), rows per tile, sets of waves per workgroup (2: the
// groups are split in halves over two sets, which needs an even group count)
// and outputs per workgroup (3: Q, K and V; 1: one of them, three times the
// workgroups).  Every form holds one workgroup per compute unit.  pass_cost: the time of one
// full pass of the form over the compute units, relative to 8 waves x 128
// rows (1000), measured at n = k = 4096 (16x16x32 f16 MFMA, 8 waves of 128
// rows: ~85 us per pass).  Small tiles cost more per output (the unpack is
// amortised over fewer rows), so the choice trades tile efficiency against
// how well the grid fills whole passes.
struct PrefillForm {
  uint32_t waves, bm, sets, outs;
};
struct PrefillFormCost {
  PrefillForm f;
  uint32_t pass_cost;
};
constexpr PrefillFormCost kPrefillForms[] = {
    {{8, 128, 1, 3}, 1000}, {{8, 96, 1, 3}, 780}, {{4, 128, 2, 3}, 555}, {{4, 96, 2, 3}, 450},
    {{4, 64, 2, 3}, 355},   {{4, 128, 1, 3}, 640}, {{4, 96, 1, 3}, 520}, {{4, 64, 1, 3}, 400}};
// s sets need a group count divisible by s; two three-output INT8 rings of
// 128-row tiles do not fit in LDS
constexpr bool prefill_form_ok(PrefillForm f, uint32_t k, uint32_t bits) {
  return f.sets == 1 || ((k / 128) % f.sets == 0 && (bits == 4 || f.bm <= 96 || f.outs == 1));
}
constexpr uint64_t prefill_wgs(PrefillForm f, uint32_t m, uint32_t n) {
  return (uint64_t)((m + f.bm - 1) / f.bm) * ((n + 16 * f.waves - 1) / (16 * f.waves)) * (f.outs == 1 ? 3 : 1);
}
// predicted time: whole passes at the full cost, a partial last pass at
// 0.7 + 0.3 x its share of the compute units (fewer workgroups contend less)
constexpr uint64_t prefill_cost(const PrefillFormCost& c, uint32_t m, uint32_t n) {
  const uint64_t wgs = prefill_wgs(c.f, m, n);
  const uint64_t full = wgs / kComputeUnits, rem = wgs % kComputeUnits;
  return c.pass_cost * (1000 * full + (rem ? 700 + 300 * rem / kComputeUnits : 0));
}
// the form with the least predicted time (the first of equals)
constexpr PrefillForm prefill_form(uint32_t m, uint32_t n, uint32_t k, uint32_t bits) {
  PrefillForm best = kPrefillForms[0].f;
  uint64_t best_cost = ~0ull;
  for (const PrefillFormCost& c : kPrefillForms) {
    if (!prefill_form_ok(c.f, k, bits)) continue;
    const uint64_t t = prefill_cost(c, m, n);
    if (t < best_cost) {
      best_cost = t;
      best = c.f;
    }
  }
  return best;
}
constexpr uint32_t kMaxN = 1u << 26;   // keeps 32-bit per-lane byte offsets in range (16 rows x N x 4 B)
constexpr uint32_t kMaxK = 1u << 24;
#ifndef KAIO_SK_MAXM
#define KAIO_SK_MAXM 64
#endif
constexpr uint32_t kDecodeMaxM = KAIO_SK_MAXM;   // the split-K kernel covers m <= this
// INT4 at 32 < m <= 64 with a group count divisible by 4 runs the tile kernel
// instead: one output per workgroup, 4 waves x 16 columns, 64-row tiles, four
// sets of waves (16 waves, four per SIMD) each over a quarter of the groups
// in a tight ring (148 KiB of LDS for the four; INT8's would not fit).  The
// four sets' independent load streams hide the latency that one group of
// lead leaves exposed.  Same-box graph replay over rotated weights, N = K =
// 4096, us (split-K -> four sets): m = 40 16.3 -> 15.3, 48 16.7 -> 15.5, 64
// 17.4 -> 15.7 (bit-identical: both split K into the same four parts); at
// m <= 32 it was slower (m = 32 11.8 -> 15.4), and at m > 64, where 64-row
// tiles double the grid, too (m = 80 20.2 -> 27.9).
constexpr bool qkv_split_k(uint32_t m, uint32_t k, uint32_t bits) {
  return m <= kDecodeMaxM && !(m > 32 && bits == 4 && (k / 128) % 4 == 0);
}
// Above kDecodeMaxM and up to kOneOutMaxM rows the tile kernel runs with one output per
// workgroup: 4 waves x 16 columns, 96-row tiles up to 96 rows and 128-row
// tiles beyond, the groups split over two sets of waves when their count is
// even.  At n = k = 4096 that is 192 workgroups where the three-output forms
// have 64; each weight word is unpacked once per tile instead of once per 32
// rows as in the split-K kernel.  Graph replay over rotated weight sets
// (us, split-K -> this form): m = 72 26.5 -> 20.3, 96 26.9 -> 20.9, 112
// 27.0 -> 22.6, 128 27.3 -> 23.3; at m <= 64 it was slower (m = 64 17.5 ->
// 18.3), and so were three-output 64-row tiles (30.3-30.8) and one-output
// 64-row tiles (32.5-32.9).  Its groups are short (32 MFMAs per wave), so
// the weights' memory latency, covered only one group ahead, bounds it.
constexpr uint32_t kOneOutMaxM = 128;
// the form of the tile kernel where qkv_split_k is false
constexpr PrefillForm tile_form(uint32_t m, uint32_t n, uint32_t k, uint32_t bits) {
  if (m <= kDecodeMaxM) return PrefillForm{4, 64, 4, 1};
  if (m <= kOneOutMaxM) return PrefillForm{4, m <= 96 ? 96u : 128u, (k / 128) % 2 == 0 ? 2u : 1u, 1};
  return prefill_form(m, n, k, bits);
}
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
constexpr uint32_t decode_bn(uint32_t m) { return m <= 32 ? 64u : 16u * KAIO_SK4_VEC; }
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
