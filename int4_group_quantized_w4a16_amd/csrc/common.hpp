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

// INT4 -> f16 times 2^-9, exact, in k order (10 VALU ops per word against
// the 12 of unpack_int4x8).
//
// Two bit operations split the sign-flipped word (q -> q + 8 in [0, 15])
// into its low nibbles and its high nibbles, each still in place within its
// byte.  For byte j one byte permute then builds the dword whose halves are
// 0x00:lo_j and 0x00:hi_j -- f16 subnormals worth (q_{2j} + 8) * 2^-24 and
// 16 (q_{2j+1} + 8) * 2^-24 -- and one packed f16 FMA with (2^15, 2^11) and
// (-2^-6, -2^-6) returns (q_{2j} * 2^-9, q_{2j+1} * 2^-9), exactly (f16
// subnormal inputs are kept: the kernels run with f16 denormals enabled).
// The results are normal f16 numbers; an MFMA over them gives 2^-9 times the
// sum over exact integers, exactly, as no product or partial sum leaves the
// f32 normal range, so multiplying by 512 * scale in the fold reproduces
// partial * scale bit for bit.
constexpr float kUnpackScaledInv = 512.0f;   // 1 / the 2^-9 factor of unpack_int4x8_scaled
__device__ __forceinline__ half8_t unpack_int4x8_scaled(uint32_t w) {
  const half2_t mul = {(_Float16)32768.0f, (_Float16)2048.0f};
  const half2_t add = {(_Float16)-0.015625f, (_Float16)-0.015625f};
  const uint32_t lo = (w ^ 0x88888888u) & 0x0F0F0F0Fu;   // low nibbles of the bytes, sign-flipped
  const uint32_t hi = (w ^ 0x88888888u) & 0xF0F0F0F0u;   // high nibbles, sign-flipped
  half8_t out;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // selector bytes: j picks byte j of lo, 4 + j byte j of hi, 0x0C a zero byte
    const uint32_t sel = 0x0C000C00u | (uint32_t)(j | ((4 + j) << 16));
    const uint32_t t = __builtin_amdgcn_perm(hi, lo, sel);
    half2_t h = __builtin_bit_cast(half2_t, t);
    h = __builtin_elementwise_fma(h, mul, add);
    out[2 * j] = h[0];
    out[2 * j + 1] = h[1];
  }
  return out;
}

// INT8 -> f16 times 2^-9, exact, in k order (the W8A16 sibling; 5 VALU ops
// per word of four values, the same cost per value as unpack_int4x8_scaled).
//
// Byte i of a word holds the signed value at k = 4r + i.  Flipping each
// byte's top bit turns q into q + 128 in [0, 255]; one byte permute per pair
// builds the dword [b_i, 0x00, b_{i+1}, 0x00], whose halves are the f16
// subnormals (q_i + 128) * 2^-24 and (q_{i+1} + 128) * 2^-24, and one packed
// f16 FMA with 2^15 and -2^-2 returns (q_i * 2^-9, q_{i+1} * 2^-9), exactly
// (8 significant bits, normal for q != 0).  As with INT4, an MFMA over these
// values is 2^-9 times the integer partial sum, exactly, and the fold's
// 512 * scale restores it bit for bit.
__device__ __forceinline__ half4_t unpack_int8x4_scaled(uint32_t w) {
  const half2_t mul = {(_Float16)32768.0f, (_Float16)32768.0f};
  const half2_t add = {(_Float16)-0.25f, (_Float16)-0.25f};
  const uint32_t u = w ^ 0x80808080u;
  // selector bytes: 0..3 pick bytes of the second operand (u), 0x0C a zero byte
  const half2_t lo = __builtin_elementwise_fma(
      __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0u, u, 0x0C010C00u)), mul, add);
  const half2_t hi = __builtin_elementwise_fma(
      __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0u, u, 0x0C030C02u)), mul, add);
  return half4_t{lo[0], lo[1], hi[0], hi[1]};
}

// One MFMA B operand (eight consecutive k of one column, times 2^-9) from
// the packed words that hold them: one INT4 word, or two INT8 words (k order).
template <int BITS>
__device__ __forceinline__ half8_t unpack_b_scaled(const uint32_t* w) {
  if constexpr (BITS == 4) {
    return unpack_int4x8_scaled(w[0]);
  } else {
    const half4_t a = unpack_int8x4_scaled(w[0]), b = unpack_int8x4_scaled(w[1]);
    return half8_t{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
}

// INT4 -> f16, exact, in nibble-interleaved order.
//
// Same exact integers as unpack_int4x8, but the eight results come out in the
// k order [0, 4, 1, 5, 2, 6, 3, 7] (nibbles i and i+4 sit 16 bits apart, so
// one bit-select builds both halves of an f16 pair).  An MFMA over these B
// values needs its A values in the same k order: see permute_x_like_int4x8.
// Cost: 4 bit-selects, 1 shift, 4 packed f16 ops per word (vs 12 ops).
__device__ __forceinline__ uint32_t nibble_pair(uint32_t w, uint32_t sel_mask, uint32_t bits) {
  // bits inside sel_mask: w with the nibble's top bit flipped (q -> q + 8);
  // bits outside: the f16 exponent pattern of 1024 (0x6400)
  return (sel_mask & (w ^ bits)) | (~sel_mask & bits);
}
__device__ __forceinline__ half8_t unpack_int4x8_interleaved(uint32_t w) {
  const half2_t lo_add = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const half2_t hi_mul = {(_Float16)0.0625f, (_Float16)0.0625f};
  const half2_t hi_add = {(_Float16)-72.0f, (_Float16)-72.0f};
  const uint32_t w8 = w >> 8;
  // (nibble i, nibble i+4) -> (1024 + q_i + 8, 1024 + q_{i+4} + 8)       for i = 0, 2
  // (nibble i, nibble i+4) -> (1024 + 16(q_i + 8), 1024 + 16(q_{i+4} + 8)) for i = 1, 3
  const half2_t p0 = __builtin_bit_cast(half2_t, nibble_pair(w, 0x000F000Fu, 0x64086408u)) + lo_add;
  const half2_t p1 = __builtin_elementwise_fma(
      __builtin_bit_cast(half2_t, nibble_pair(w, 0x00F000F0u, 0x64806480u)), hi_mul, hi_add);
  const half2_t p2 = __builtin_bit_cast(half2_t, nibble_pair(w8, 0x000F000Fu, 0x64086408u)) + lo_add;
  const half2_t p3 = __builtin_elementwise_fma(
      __builtin_bit_cast(half2_t, nibble_pair(w8, 0x00F000F0u, 0x64806480u)), hi_mul, hi_add);
  const uint4 d = {__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                   __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
  return __builtin_bit_cast(half8_t, d);
}

// Reorders eight consecutive f16 (k offsets 0..7) into [0, 4, 1, 5, 2, 6, 3, 7],
// the k order of unpack_int4x8_interleaved.
__device__ __forceinline__ half8_t permute_x_like_int4x8(uint4 v) {
  const uint4 o = {(v.x & 0xFFFFu) | (v.z << 16), (v.x >> 16) | (v.z & 0xFFFF0000u),
                   (v.y & 0xFFFFu) | (v.w << 16), (v.y >> 16) | (v.w & 0xFFFF0000u)};
  return __builtin_bit_cast(half8_t, o);
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

// Tile (m, n) of remapped id t for an mtiles x ntiles grid.  Consecutive
// ids run concurrently on one XCD; they are walked in SM x SN super-blocks
// (SM row blocks x SN column blocks) so that the tiles resident on an XCD
// share both x row blocks and weight column blocks in its L2 instead of
// spanning every row block of x.
template <uint32_t SM, uint32_t SN>
__device__ __forceinline__ void tile_at(uint32_t t, uint32_t mtiles, uint32_t ntiles, uint32_t& tm, uint32_t& tn) {
  if (mtiles % SM == 0 && ntiles % SN == 0) {
    const uint32_t per = SM * SN;
    const uint32_t blk = t / per, in = t % per;
    const uint32_t bm = mtiles / SM;                 // super-blocks along m
    tm = (blk % bm) * SM + in % SM;
    tn = (blk / bm) * SN + in / SM;
  } else {
    tm = t % mtiles;
    tn = t / mtiles;
  }
}

// Tile (m, n) of workgroup b of nb for an mtiles x ntiles grid.
template <uint32_t SM, uint32_t SN>
__device__ __forceinline__ void tile_of(uint32_t b, uint32_t nb, uint32_t mtiles, uint32_t ntiles,
                                        uint32_t& tm, uint32_t& tn) {
  tile_at<SM, SN>(xcd_remap(b, nb), mtiles, ntiles, tm, tn);
}

}  // namespace kaio
