// Internal helpers shared by the gfx950 kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kaio {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kGroup = 128;  // quantization group along K (locked)

// ---------------------------------------------------------------------------
// INT4 -> f16, exact.
//
// A packed word holds eight signed 4-bit values; nibble i (bits 4i..4i+3)
// is the weight at k = 8r + i.  Byte j therefore carries k = 2j (low nibble)
// and k = 2j+1 (high nibble).  For each byte we build, with one byte
// permute, the dword [b, 0x64, b, 0x64]; masking keeps the low nibble in the
// low half and the high nibble (still shifted by 4) in the high half, and
// flipping bit 3 of each nibble turns the two's-complement value q into
// q + 8 in [0, 15].  With 0x64 as the high byte the halves read as the f16
// numbers 1024 + (q_lo + 8) and 1024 + 16 * (q_hi + 8); one packed f16 FMA
// with (1, 1/16) and (-1032, -72) returns (q_lo, q_hi).  Every step is exact.
// The eight results come out in k order, so the MFMA B operand built from one
// word matches an A operand of eight consecutive k.
// ---------------------------------------------------------------------------
__device__ __forceinline__ half8_t unpack_int4x8(uint32_t w) {
  const half2_t mul = {(_Float16)1.0f, (_Float16)0.0625f};
  const half2_t add = {(_Float16)-1032.0f, (_Float16)-72.0f};
  half8_t out;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // selector bytes: 0..3 pick bytes of the second operand (w), 4 picks byte 0
    // of the first operand (0x64646464)
    const uint32_t sel = 0x04000400u | (uint32_t)(j * 0x00010001u);
    uint32_t t = __builtin_amdgcn_perm(0x64646464u, w, sel);
    t = (t & 0xFFF0FF0Fu) ^ 0x00800008u;
    half2_t h = __builtin_bit_cast(half2_t, t);
    h = __builtin_elementwise_fma(h, mul, add);
    out[2 * j] = h[0];
    out[2 * j + 1] = h[1];
  }
  return out;
}

__device__ __forceinline__ floatx4 mfma16x16x32(half8_t a, half8_t b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float h2f(uint16_t bits) {
  return (float)__builtin_bit_cast(_Float16, bits);
}

// XCD-aware tile order.  Workgroups are dealt round-robin to the 8 XCDs
// (workgroup b runs on XCD b % 8); remapping gives each XCD one contiguous
// range of tiles, so tiles that share operands also share an L2.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t b, uint32_t nb) {
  constexpr uint32_t kXcd = 8;
  const uint32_t per = nb / kXcd;           // full rounds
  const uint32_t full = per * kXcd;
  if (b >= full) return b;                  // ragged last round keeps its order
  return (b % kXcd) * per + b / kXcd;
}

}  // namespace kaio
