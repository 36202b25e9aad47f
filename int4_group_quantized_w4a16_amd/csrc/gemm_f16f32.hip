// Dense f16 x f16 -> f32 matmul, C = A . B, and its backward.
//
// Operation: kaio-candle 0.2.0, src/matmul_tc_async.rs (module doc;
// MatmulTcAsyncOp::cuda_fwd: A [m,k] and B [k,n] f16, a zeroed [m,n] f32
// output that the kernel writes; MatmulTcAsyncOp::bwd: the f32 output
// gradient cast to f16, grad_a = grad . B^T and grad_b = A^T . grad through
// the forward kernel, each result cast to f16).  The pages stage tiles
// global -> shared with cp.async on sm_80+; here the main path moves them
// global -> LDS with gfx950's direct loads, the fallback through registers.
//
// gfx950 design
// -------------
// * Direct-to-LDS path: workgroup = 8 waves, tile 256 x 256; each wave owns a
//   128 x 64 sub-tile = 8 x 4 v_mfma_f32_16x16x32_f16 accumulators (128 f32
//   per lane, held in the accumulation registers), so two waves share each
//   SIMD and one issues MFMAs while the other waits at a barrier or on an LDS
//   read (the 4-wave form with 128 x 128 sub-tiles, one wave per SIMD and the
//   least LDS traffic per MFMA, remains as WN = 2: 0.4-2% slower at
//   4096^3, 14% slower when the grid covers half the compute units).
//   The register-staged fallback keeps 4 waves of 128 x 128.
// * Main path (reduction % 64 == 0, strides % 8 == 0): both operand tiles
//   land in LDS via 16-byte direct loads into four 32-k half-stage buffers;
//   each half-stage of MFMAs reads the next fragments and loads the half
//   that will be needed two half-stages later, one barrier per half-stage.
//   Each operand is staged in its own layout: reduction-contiguous (plain
//   16-byte fragment reads) or index-contiguous (transposing LDS reads), so
//   one kernel template serves the forward product and both backward
//   products without transposed copies.
// * Fallback (any other shape): forward tiles go global -> registers -> LDS,
//   B transposed in registers (8x8 blocks of 16-bit values) so LDS holds B^T;
//   the backward products use a strided one-output-per-thread kernel.
// * Epilogue: f32 (forward) or f16 (backward, round to nearest even) stores
//   straight from the accumulators.

#include "common.hpp"
#include "launch.hpp"

#include <mutex>
#include <type_traits>

namespace kaio {
namespace {

constexpr int BM = kGemmBM;      // 256
constexpr int BN = kGemmBN;      // 256
constexpr int BK = 64;
constexpr int THREADS = 256;
constexpr int KCH = BK / 8;      // 16-byte chunks per tile row
constexpr int WT = 128;          // wave tile edge
constexpr int TT = WT / 16;      // 16x16 tiles per wave edge

struct alignas(16) SmemGemm {
  uint4 a[BM * KCH];   // 32 KiB, [m][k-chunk] swizzled
  uint4 b[BN * KCH];   // 32 KiB, [n][k-chunk] swizzled (B transposed)
};

__device__ __forceinline__ uint32_t lo_pair(uint32_t r0, uint32_t r1) { return (r0 & 0xFFFFu) | (r1 << 16); }
__device__ __forceinline__ uint32_t hi_pair(uint32_t r0, uint32_t r1) { return (r0 >> 16) | (r1 & 0xFFFF0000u); }

__device__ __forceinline__ void store_out(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_out(uint16_t* p, float v) { *p = __builtin_bit_cast(uint16_t, (_Float16)v); }

// How an operand's 8-element chunks are read.
//   kLoadAligned: ld % 8 == 0 and the contiguous extent % 8 == 0: a chunk is
//     wholly inside or outside the matrix and starts 16 bytes aligned.
//   kLoadClamped: contiguous extent >= 8, any ld: every chunk is one 16-byte
//     load (2-byte aligned; gfx950 runs with unaligned access enabled and the
//     compiler emits a single dwordx4 load) from a start clamped into the
//     matrix; fix8 then moves the wanted elements into place and zeroes those
//     past the end, once the data has landed.  No load sits under a branch,
//     so the next stage's loads stay in flight over the MFMAs.
//   kLoadElement: element by element (contiguous extent < 8).
constexpr int kLoadElement = 0, kLoadClamped = 1, kLoadAligned = 2;

// Eight consecutive 16-bit elements base[outer * ld + inner .. + 7]; under
// kLoadAligned and kLoadElement, elements at or past (outer_lim, inner_lim)
// read as zero; under kLoadClamped the raw load of the clamped chunk, which
// fix8 with the same indices turns into that.
template <int kMode>
__device__ __forceinline__ uint4 load8(const uint16_t* base, size_t ld, uint32_t outer, uint32_t outer_lim,
                                       uint32_t inner, uint32_t inner_lim) {
  if constexpr (kMode == kLoadClamped) {
    const uint32_t o = outer < outer_lim ? outer : outer_lim - 1;
    const uint32_t st = inner + 8 <= inner_lim ? inner : inner_lim - 8;
    uint4 v;
    __builtin_memcpy(&v, base + (size_t)o * ld + st, 16);
    return v;
  }
  if (outer >= outer_lim) return uint4{0u, 0u, 0u, 0u};
  if constexpr (kMode == kLoadAligned) {
    if (inner >= inner_lim) return uint4{0u, 0u, 0u, 0u};
    return *reinterpret_cast<const uint4*>(base + (size_t)outer * ld + inner);
  }
  uint16_t h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = (inner + i < inner_lim) ? base[(size_t)outer * ld + inner + i] : (uint16_t)0;
  return uint4{h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16),
               h[4] | ((uint32_t)h[5] << 16), h[6] | ((uint32_t)h[7] << 16)};
}

// The chunk (outer, inner) from what load8<kLoadClamped> read for it: unchanged
// inside the matrix; past the end of a row the load started at inner_lim - 8,
// so the wanted elements sit inner + 8 - inner_lim places up and are shifted
// down, zeros filling the positions past inner_lim.
__device__ __forceinline__ uint4 fix8(uint4 v, uint32_t outer, uint32_t outer_lim, uint32_t inner,
                                      uint32_t inner_lim) {
  if (outer >= outer_lim || inner >= inner_lim) return uint4{0u, 0u, 0u, 0u};
  if (inner + 8 <= inner_lim) return v;
  const uint32_t sh = 16u * (inner + 8 - inner_lim);   // 16 .. 112 bits
  uint64_t lo = v.x | ((uint64_t)v.y << 32), hi = v.z | ((uint64_t)v.w << 32);
  if (sh >= 64) {
    lo = hi >> (sh - 64);
    hi = 0;
  } else {
    lo = (lo >> sh) | (hi << (64 - sh));
    hi >>= sh;
  }
  return uint4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
}

// LDS swizzle of an operand tile [256 indices][8 reduction chunks]: chunk kc
// of index i sits in slot i*8 + (kc ^ swz(i)).  An operand staged from
// reduction-contiguous rows is written one row of 8 chunks per 8 lanes
// (i & 7 keeps those apart and the 16-row fragment reads too); one staged by
// transposing 8x8 blocks in registers is written 8 rows at a time, the same
// chunk of rows 8 apart from neighbouring lanes ((i ^ (i >> 3)) & 7 puts
// them in distinct bank groups, as it does the fragment reads).
template <bool kTransposed>
__device__ __forceinline__ uint32_t tile_swz(uint32_t i) { return kTransposed ? ((i ^ (i >> 3)) & 7) : (i & 7); }

// Register-staged product for shapes the direct-to-LDS kernel does not take:
// C[Mo, No] = sum over R of A-operand x B-operand, f32 accumulation, OutT
// float (f32 out) or uint16_t (f16 out, round to nearest even).
//   kATr = false: A(i, r) at A[i * lda + r] (reduction contiguous);
//          true:  A(i, r) at A[r * lda + i] (index contiguous).
//   kBTr = true:  B(r, j) at B[r * ldb + j] (index contiguous);
//          false: B(r, j) at B[j * ldb + r] (reduction contiguous).
// A reduction-contiguous operand is staged in 16-byte chunks of 8 reduction
// elements; an index-contiguous one in 8 x 8 blocks transposed in registers,
// so that LDS holds both operands as [index][reduction] and every fragment is
// one 16-byte read.  The forward product is <false, true, float>; the
// backward products <false, false, f16> (grad_a) and <true, true, f16>
// (grad_b).  kAMode / kBMode: how each operand's chunks are read (kLoad*).
template <int kAMode, int kBMode, bool kATr, bool kBTr, typename OutT>
__global__ void __launch_bounds__(THREADS, 1)
gemm_reg_kernel(const uint16_t* __restrict__ A, uint32_t lda, const uint16_t* __restrict__ B, uint32_t ldb,
                OutT* __restrict__ C, uint32_t Mo, uint32_t No, uint32_t R, uint32_t mtiles) {
  __shared__ SmemGemm sm;

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t wave = tid >> 6;
  const uint32_t kb = lane >> 4;
  const uint32_t l16 = lane & 15;
  const uint32_t wm = wave >> 1, wn = wave & 1;

  const uint32_t bidx = xcd_remap(blockIdx.x, gridDim.x);
  const uint32_t m0 = (bidx % mtiles) * BM;
  const uint32_t n0 = (bidx / mtiles) * BN;

  // Staging assignment.  Reduction-contiguous operand: chunk c = i*256 + tid
  // -> index c / 8, reduction chunk c % 8.  Index-contiguous operand: thread
  // -> 8x8 block of index block ib = tid % 32 and reduction block kq = tid / 32.
  const uint32_t ib = tid & 31, kq = tid >> 5;

  uint4 ra[8], rb[8];
  // one operand's next tile into registers: base, stride, first index, index count
  auto load_op = [&](auto tr, auto al, uint4 (&reg)[8], const uint16_t* base, uint32_t ld, uint32_t i0,
                     uint32_t ilim, uint32_t k0) {
    constexpr int kAl = decltype(al)::value;
    if constexpr (decltype(tr)::value) {
#pragma unroll
      for (int i = 0; i < 8; ++i) reg[i] = load8<kAl>(base, ld, k0 + kq * 8 + i, R, i0 + ib * 8, ilim);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t c = i * THREADS + tid;
        const uint32_t row = c >> 3, kc = c & 7;
        const uint32_t gi = i0 + row < ilim ? i0 + row : ilim - 1;   // indices past the end: any valid one
        reg[i] = load8<kAl>(base, ld, gi, ilim, k0 + kc * 8, R);
      }
    }
  };
  auto store_op = [&](auto tr, const uint4 (&reg)[8], uint4* dst) {
    constexpr bool kT = decltype(tr)::value;
    if constexpr (kT) {
      // transpose the 8x8 block: out[j] = index j of the block, 8 consecutive reduction elements
      uint32_t d[8][4];
#pragma unroll
      for (int i = 0; i < 8; ++i) { d[i][0] = reg[i].x; d[i][1] = reg[i].y; d[i][2] = reg[i].z; d[i][3] = reg[i].w; }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int qd = j >> 1;
        uint4 o;
        if (j & 1) {
          o = uint4{hi_pair(d[0][qd], d[1][qd]), hi_pair(d[2][qd], d[3][qd]),
                    hi_pair(d[4][qd], d[5][qd]), hi_pair(d[6][qd], d[7][qd])};
        } else {
          o = uint4{lo_pair(d[0][qd], d[1][qd]), lo_pair(d[2][qd], d[3][qd]),
                    lo_pair(d[4][qd], d[5][qd]), lo_pair(d[6][qd], d[7][qd])};
        }
        const uint32_t idx = ib * 8 + j;
        dst[idx * KCH + (kq ^ tile_swz<true>(idx))] = o;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t c = i * THREADS + tid;
        const uint32_t row = c >> 3, kc = c & 7;
        dst[row * KCH + (kc ^ tile_swz<false>(row))] = reg[i];
      }
    }
  };
  using ATr = std::integral_constant<bool, kATr>;
  using BT = std::integral_constant<bool, kBTr>;
  using AMode = std::integral_constant<int, kAMode>;
  using BMode = std::integral_constant<int, kBMode>;
  auto load_tiles = [&](uint32_t k0) {
    load_op(ATr{}, AMode{}, ra, A, lda, m0, Mo, k0);
    load_op(BT{}, BMode{}, rb, B, ldb, n0, No, k0);
  };
  // the clamped loads' fixes, same indices as load_op, after the data landed;
  // only a stage that reaches past the reduction, or an index-contiguous
  // operand's last tile, holds chunks to fix (a uniform branch elsewhere)
  auto fix_op = [&](auto tr, auto mode, uint4 (&reg)[8], uint32_t i0, uint32_t ilim, uint32_t k0) {
    if constexpr (decltype(mode)::value == kLoadClamped) {
      static_assert(BM == 32 * 8 && BN == 32 * 8, "an index-contiguous tile is 32 lanes of 8 indices");
      if (k0 + BK <= R && (!decltype(tr)::value || i0 + 32 * 8 <= ilim)) return;
      if constexpr (decltype(tr)::value) {
#pragma unroll
        for (int i = 0; i < 8; ++i) reg[i] = fix8(reg[i], k0 + kq * 8 + i, R, i0 + ib * 8, ilim);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) reg[i] = fix8(reg[i], 0, 1, k0 + ((i * THREADS + tid) & 7) * 8, R);
      }
    }
  };

  floatx4 acc[TT][TT];
#pragma unroll
  for (int r = 0; r < TT; ++r)
#pragma unroll
    for (int c = 0; c < TT; ++c) acc[r][c] = floatx4{0.f, 0.f, 0.f, 0.f};

  const uint32_t nk = (R + BK - 1) / BK;
  if (nk > 0) load_tiles(0);
  for (uint32_t it = 0; it < nk; ++it) {
    __syncthreads();            // previous tile fully consumed
    fix_op(ATr{}, AMode{}, ra, m0, Mo, it * BK);
    fix_op(BT{}, BMode{}, rb, n0, No, it * BK);
    store_op(ATr{}, ra, sm.a);
    store_op(BT{}, rb, sm.b);
    __syncthreads();            // tile visible
    if (it + 1 < nk) load_tiles((it + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      const uint32_t kc = ks * 4 + kb;
      half8_t bf[TT];
#pragma unroll
      for (int c = 0; c < TT; ++c) {
        const uint32_t n = wn * WT + c * 16 + l16;
        bf[c] = __builtin_bit_cast(half8_t, sm.b[n * KCH + (kc ^ tile_swz<kBTr>(n))]);
      }
#pragma unroll
      for (int r = 0; r < TT; ++r) {
        const uint32_t row = wm * WT + r * 16 + l16;
        const half8_t af = __builtin_bit_cast(half8_t, sm.a[row * KCH + (kc ^ tile_swz<kATr>(row))]);
#pragma unroll
        for (int c = 0; c < TT; ++c) acc[r][c] = mfma16x16x32(af, bf[c], acc[r][c]);
      }
    }
  }

#pragma unroll
  for (int r = 0; r < TT; ++r)
#pragma unroll
    for (int c = 0; c < TT; ++c) {
      const uint32_t gc = n0 + wn * WT + c * 16 + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t gr = m0 + wm * WT + r * 16 + 4 * kb + i;
        if (gr < Mo && gc < No) store_out(C + (size_t)gr * No + gc, acc[r][c][i]);
      }
    }
}

// ---------------------------------------------------------------------------
// DMA path (k % 64 == 0, n % 8 == 0): both tiles go global -> LDS with
// 16-byte direct loads in their natural layouts, two stages deep, no
// registers and no VALU on the way.  A fragments are plain 16-byte LDS reads;
// B fragments come from gfx950's transposing LDS read (ds_read_b64_tr_b16):
// within each 16-lane group, lane i receives element i % 4 of the 8-byte
// chunks that lanes 4j + i / 4 address, j = 0..3.  Lane a of a group
// addresses row k0 + a / 4, columns 4(a % 4) .. +3 of the [k][n] tile, so
// lane i gets B[k0 + j][i] for j = 0..3: four consecutive k of its column,
// and two such reads make its eight-k MFMA B operand.
//   A tile [256][64]: chunk kc of row r at slot r*8 + (kc ^ (r & 7)).
//   B tile [64][256]: chunk c of k-row r at slot r*32 + (c ^ tr_swz(r)).
// ---------------------------------------------------------------------------
#define KAIO_GEMM_LDS(p) ((__attribute__((address_space(3))) void*)(p))
#define KAIO_GEMM_GLOBAL(p) ((__attribute__((address_space(1))) const void*)(p))
typedef short short4_t __attribute__((ext_vector_type(4)));

#ifndef KAIO_GEMM_SM
#define KAIO_GEMM_SM 4
#endif
#ifndef KAIO_GEMM_SN
#define KAIO_GEMM_SN 8
#endif
constexpr int DBK = 64;
// word 3 of a raw buffer descriptor on the gfx9 family: 32-bit data format,
// no swizzle, no index stride
constexpr int kBufferFlags = 0x00020000;
constexpr int HSLOTS = 1024;   // 16-byte slots of one operand's 32-k half-stage tile (256 x 32 f16)
// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8): nothing outstanding
constexpr int kWait0 = 0x0070;
// s_waitcnt immediate for "at most vm loads outstanding, no LDS read"
constexpr int wait_vm_imm(int vm) { return (vm & 15) | ((vm >> 4) << 14) | 0x70; }

__device__ __forceinline__ const char* sgpr_ptr(const char* p) {
  asm volatile("" : "+s"(p));
  return p;
}
__device__ __forceinline__ uint32_t vgpr_u32(uint32_t o) {
  asm volatile("" : "+v"(o));
  return o;
}

// Staging of one operand on the direct-to-LDS path.  The LDS holds four
// half-stage buffers (stage s % 2, 32-k half h), each with an A part and a B
// part of 1024 16-byte slots.  Each operand tile half covers 256 output
// indices (rows of the product for the A side, columns for the B side) by 32
// reduction indices.
//   kTr = false: stored [index][reduction] (reduction contiguous, row stride
//     ld): LDS [256][4 chunks], chunk kc of index row i at slot
//     i*4 + (kc ^ idx_swz(i)); a fragment is one 16-byte read.
//   kTr = true: stored [reduction][index] (index contiguous, row stride ld):
//     LDS [32][32 chunks], chunk c of reduction row r at slot r*32 + (c ^ tr_swz(r));
//     a fragment is two transposing reads.
// Chunk swizzle of the index-contiguous layout.  One transposing read of a
// wave touches k-rows kb*8 + {0..3} (+4 for the second read) for kb = 0..3,
// 32 bytes (two chunks) of each; the hardware serves 32 lanes (two kb) per
// pass.  2(r & 3) moves rows r and r+1..r+3 to different chunk pairs, and
// 8((r >> 3) & 1) moves rows kb*8 + j and (kb+1)*8 + j apart, so the 16 chunk
// slots of one pass fall in 16 distinct 16-byte bank groups.  (Without the
// second term rows j and 8 + j shared their banks: two-way conflicts on
// every transposing read.)
__device__ __forceinline__ uint32_t tr_swz(uint32_t r) { return (2 * (r & 3)) ^ (8 * ((r >> 3) & 1)); }
// Chunk swizzle of the reduction-contiguous layout.  A fragment read has
// lanes 16j + l read index rows i0 + l (l < 16), chunk j, and the LDS serves
// 16-byte reads eight lanes at a time over 128 bytes of banks (counters: the
// earlier swizzle (i >> 2) & 3, distinct over 16 lanes and 256 bytes but not
// over 8 and 128, read two conflict cycles per instruction).  This one puts
// the 8 rows of every aligned 8-lane group in 8 distinct 16-byte bank groups
// mod 128 bytes, and the 16 rows of every 16-lane group in 16 distinct ones
// mod 256 bytes.
__device__ __forceinline__ uint32_t idx_swz(uint32_t i) { return ((i >> 1) & 3) ^ (((i >> 3) & 1) * 3); }

template <bool kTr>
struct DmaOperand {
  // byte offset, within a half-stage's source window, of this lane's load i
  // (0 .. 1024 / (64 * NW) - 1) of a workgroup of NW waves
  template <int NW>
  __device__ static uint32_t lane_offset(int i, uint32_t wave, uint32_t lane, uint32_t idx0, uint32_t nidx,
                                         uint32_t ld) {
    const uint32_t s = (i * NW + wave) * 64 + lane;
    if (!kTr) {
      const uint32_t r = s >> 2, kc = (s & 3) ^ idx_swz(r);
      const uint32_t rc = (idx0 + r < nidx) ? r : nidx - 1 - idx0;   // rows past the end repeat a valid one
      return (rc * ld + kc * 8) * 2;
    }
    const uint32_t r = s >> 5, c = (s & 31) ^ tr_swz(r);
    const uint32_t cc = (idx0 + c * 8 < nidx) ? c * 8 : nidx - 8 - idx0;   // likewise for 8-index chunks
    return (r * ld + cc) * 2;
  }
  // reduction offset, within a 32-k half, of the first element of this lane's load i
  template <int NW>
  __device__ static uint32_t lane_reduction(int i, uint32_t wave, uint32_t lane) {
    const uint32_t s = (i * NW + wave) * 64 + lane;
    if (!kTr) {
      const uint32_t r = s >> 2;
      return ((s & 3) ^ idx_swz(r)) * 8;   // an 8-element chunk of one index row
    }
    return s >> 5;                            // one reduction row, 8 indices
  }
  __device__ static const char* tile_base(const uint16_t* p, uint32_t idx0, uint32_t ld) {
    return reinterpret_cast<const char*>(kTr ? p + idx0 : p + (size_t)idx0 * ld);
  }
  // bytes between the sources of consecutive 32-k halves
  __device__ static size_t half_stride(uint32_t ld) { return kTr ? (size_t)32 * ld * 2 : (size_t)32 * 2; }
  // lane part of the fragment index for 16-wide tile t of the wave block at index w0
  __device__ static uint32_t lane_index(uint32_t w0, uint32_t l16) { return w0 + (kTr ? 4 * (l16 & 3) : l16); }
  // The fragment for index `idx` (lane_index + 16 t) from a half-stage buffer.
  // The buffer pointer is restrict-qualified: that tells the compiler the read
  // does not touch the buffers the loads in flight are writing, so it does not
  // make the read wait for them.
  __device__ static half8_t frag(const char* __restrict__ st, uint32_t idx, uint32_t kb, uint32_t l16) {
    if (!kTr) {
      const uint4* t = reinterpret_cast<const uint4*>(st);
      return __builtin_bit_cast(half8_t, t[idx * 4 + (kb ^ idx_swz(idx))]);
    }
    // transposing read: within each 16-lane group, lane i receives element
    // i % 4 of the 8-byte chunks that lanes 4j + i / 4 address (j = 0..3).
    // Lane a addresses reduction row k0 + a / 4 at indices 4(a % 4) .. +3 of
    // its 16-wide tile, so lane i gets four consecutive reduction values of
    // its own index; two reads (k0 and k0 + 4) make the eight of a fragment.
    short4_t h[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const uint32_t k = kb * 8 + (l16 >> 2) + 4 * hf;
      const uint32_t off = (k * 32 + ((idx >> 3) ^ tr_swz(k))) * 16 + ((idx >> 2) & 1) * 8;
      h[hf] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(st + off));
    }
    return __builtin_bit_cast(half8_t, (short __attribute__((ext_vector_type(8)))){
        h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]});
  }
};

template <int TM, int TN>
struct GemmFrags {
  half8_t a[TM], b[TN];
};

// The accumulating MFMAs of the direct-to-LDS kernel are issued through asm
// with the accumulator tied in place in the accumulation registers.  With the
// builtin, the compiler picks the form whose result register differs from the
// accumulator input, so every accumulator moves each step and is copied back
// at the loop edge: 100-300 register copies per 128 MFMAs, which cost more
// than the DMA and LDS work of the stage.
__device__ __forceinline__ void mfma_inplace(floatx4& acc, const half8_t& a, const half8_t& b) {
  asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// The asm MFMAs are invisible to the compiler's hazard tracking, which covers
// the other cases here: their A/B operands only ever come from LDS reads
// (waited on through lgkmcnt, which the compiler does track for asm operands).
// What remains are the VALU writes that zero the accumulators before the first
// MFMA reads them, and the MFMA writes before the epilogue reads the results.
// Each row of accumulators passes through an asm that takes it as an in/out
// operand and waits 2 * (NOP + 1) cycles, so no access to a row can move
// across its wait, and the wait exceeds what an 8-pass MFMA needs.
template <int NOP, int TM, int TN>
__device__ __forceinline__ void hazard_guard(floatx4 (&acc)[TM][TN]) {
  static_assert(TN == 8 || TN == 4, "one asm operand per accumulator of a row");
#pragma unroll
  for (int r = 0; r < TM; ++r) {
    if constexpr (TN == 8)
      asm volatile("s_nop %8\n\ts_nop %8"
                   : "+a"(acc[r][0]), "+a"(acc[r][1]), "+a"(acc[r][2]), "+a"(acc[r][3]),
                     "+a"(acc[r][4]), "+a"(acc[r][5]), "+a"(acc[r][6]), "+a"(acc[r][7])
                   : "i"(NOP));
    else
      asm volatile("s_nop %4\n\ts_nop %4"
                   : "+a"(acc[r][0]), "+a"(acc[r][1]), "+a"(acc[r][2]), "+a"(acc[r][3])
                   : "i"(NOP));
  }
}

// C[Mo, No] = sum over R of A-operand x B-operand, f32 accumulation; OutT is
// float (f32 out) or uint16_t (f16 out, rounded to nearest even).  A is read
// through DmaOperand<kATr> with row stride lda, B through DmaOperand<kBTr>
// with row stride ldb.  Needs the strides and, for a transposed operand, its
// index count multiples of 8, and R % 64 == 0 -- or, with kRagged, any R
// (R % 8 == 0 for an operand stored reduction-contiguous): the last stage's
// chunks past R are then zero.  A lane whose chunk starts at or past R
// points its direct load past the end of the descriptor's range, and a
// buffer load out of range returns zeros, which land in LDS like data.  No
// load is skipped, so every wave still issues exactly 2 * LPL loads per half-stage
// and the fixed vmcnt waits below stay exact.
//
// WN = waves along the tile's columns: 2 (4 waves, 128 x 128 wave tiles, one
// wave per SIMD) or 4 (8 waves, 128 x 64 wave tiles, two per SIMD).
template <bool kATr, bool kBTr, typename OutT, bool kRagged, int WN>
__global__ void __launch_bounds__(128 * WN, 1)
gemm_dma_kernel(const uint16_t* __restrict__ A, uint32_t lda, const uint16_t* __restrict__ B, uint32_t ldb,
                OutT* __restrict__ C, uint32_t Mo, uint32_t No, uint32_t R, uint32_t mtiles, uint32_t ntiles) {
  static_assert(WN == 2 || WN == 4, "waves along n");
  constexpr int NW = 2 * WN;                 // waves
  constexpr int LPL = HSLOTS / (64 * NW);    // direct loads per lane per operand per half-stage
  constexpr int TM = WT / 16;                // 16x16 tiles per wave along m (128 rows)
  constexpr int WTN = BN / WN;               // wave tile columns
  constexpr int TN = WTN / 16;
  constexpr int kWaitHalves = wait_vm_imm(2 * 2 * LPL);   // two half-stages of loads in flight
  using OA = DmaOperand<kATr>;
  using OB = DmaOperand<kBTr>;
  using Frags = GemmFrags<TM, TN>;
  extern __shared__ uint4 smem[];
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t kb = lane >> 4, l16 = lane & 15;
  const uint32_t wm = wave / WN, wn = wave % WN;

  uint32_t tm, tn;
  tile_of<KAIO_GEMM_SM, KAIO_GEMM_SN>(blockIdx.x, gridDim.x, mtiles, ntiles, tm, tn);
  const uint32_t m0 = tm * BM, n0 = tn * BN;

  uint32_t aoff[LPL], boff[LPL], ared[LPL], bred[LPL];
#pragma unroll
  for (int i = 0; i < LPL; ++i) {
    aoff[i] = OA::template lane_offset<NW>(i, wave, lane, m0, Mo, lda);
    boff[i] = OB::template lane_offset<NW>(i, wave, lane, n0, No, ldb);
    ared[i] = OA::template lane_reduction<NW>(i, wave, lane);
    bred[i] = OB::template lane_reduction<NW>(i, wave, lane);
  }
  // kRagged: descriptors span 2 GiB (every in-bounds lane offset is below
  // 2^31, by the host-side size limits); kOutOfRange lies past that
  constexpr int kRange = kRagged ? 0x7FFFFFF0 : -1;
  constexpr uint32_t kOutOfRange = 0x80000000u;
  const char* abase = OA::tile_base(A, m0, lda);
  const char* bbase = OB::tile_base(B, n0, ldb);
  const size_t ahalf = OA::half_stride(lda), bhalf = OB::half_stride(ldb);

  // half-stage buffer of stage kt, half h (A part first, B part HSLOTS later)
  auto hbuf = [&](uint32_t kt, uint32_t h) { return smem + ((kt & 1) * 2 + h) * (2 * HSLOTS); };
  // load j (0..LPL-1: A chunks, LPL..2LPL-1: B chunks) of this lane's share of half h of
  // stage kt.  The buffer form of the direct-to-LDS load is used, not the
  // global one: while a global (FLAT-encoded) load is pending the compiler can
  // no longer order the LDS counter and turns every wait for a fragment read
  // into a full wait.  The descriptor is rebuilt per half-stage from its
  // 64-bit base, so the 32-bit lane offsets never overflow; its range is
  // unlimited (every offset is in bounds by construction).
  auto issue_one = [&](uint32_t kt, uint32_t h, int j) {
    uint4* st = hbuf(kt, h);
    const uint32_t hk = 2 * kt + h;   // 32-k half index
    if (j < LPL) {
      uint32_t off = aoff[j];
      if (kRagged && 32 * hk + ared[j] >= R) off = kOutOfRange;
      const __amdgpu_buffer_rsrc_t r =
          __builtin_amdgcn_make_buffer_rsrc((void*)sgpr_ptr(abase + hk * ahalf), 0, kRange, kBufferFlags);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, KAIO_GEMM_LDS(st + (j * NW + wave) * 64), 16,
                                               vgpr_u32(off), 0, 0, 0);
    } else {
      uint32_t off = boff[j - LPL];
      if (kRagged && 32 * hk + bred[j - LPL] >= R) off = kOutOfRange;
      const __amdgpu_buffer_rsrc_t r =
          __builtin_amdgcn_make_buffer_rsrc((void*)sgpr_ptr(bbase + hk * bhalf), 0, kRange, kBufferFlags);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, KAIO_GEMM_LDS(st + HSLOTS + ((j - LPL) * NW + wave) * 64), 16,
                                               vgpr_u32(off), 0, 0, 0);
    }
  };
  auto issue_half = [&](uint32_t kt, uint32_t h) {
#pragma unroll
    for (int j = 0; j < 2 * LPL; ++j) issue_one(kt, h, j);
  };

  floatx4 acc[TM][TN];
#pragma unroll
  for (int r = 0; r < TM; ++r)
#pragma unroll
    for (int c = 0; c < TN; ++c) acc[r][c] = floatx4{0.f, 0.f, 0.f, 0.f};

  hazard_guard<4>(acc);
  const uint32_t ai0 = OA::lane_index(wm * WT, l16), bi0 = OB::lane_index(wn * WTN, l16);
  auto load_frags = [&](const uint4* hb, Frags& f) {
    const char* as = reinterpret_cast<const char*>(hb);
    const char* bs = reinterpret_cast<const char*>(hb + HSLOTS);
#pragma unroll
    for (int c = 0; c < TN; ++c) f.b[c] = OB::frag(bs, bi0 + c * 16, kb, l16);
#pragma unroll
    for (int r = 0; r < TM; ++r) f.a[r] = OA::frag(as, ai0 + r * 16, kb, l16);
  };
  // The MFMAs on fragments f, row by row, with the reads of the next
  // fragments nf (from half-stage buffer nb) spread between the rows: all B
  // fragments during rows 0-3, the A fragment of row r after row r.  Every
  // read then has at least a row of MFMAs (128 cycles) before its use, and no
  // wait ever covers a read issued just before it.  The 8 direct loads of
  // half h of stage kt go between the rows too, one per row.
  auto mma_read = [&](const Frags& f, const uint4* nb, Frags& nf, uint32_t kt, uint32_t h) {
    const char* as = reinterpret_cast<const char*>(nb);
    const char* bs = reinterpret_cast<const char*>(nb + HSLOTS);
#pragma unroll
    for (int r = 0; r < TM; ++r) {
#pragma unroll
      for (int c = 0; c < TN; ++c) mfma_inplace(acc[r][c], f.a[r], f.b[c]);
      if (r < 2 * LPL) issue_one(kt, h, r);
      if (r < TN / 2) {
        nf.b[2 * r] = OB::frag(bs, bi0 + 2 * r * 16, kb, l16);
        nf.b[2 * r + 1] = OB::frag(bs, bi0 + (2 * r + 1) * 16, kb, l16);
      }
      nf.a[r] = OA::frag(as, ai0 + r * 16, kb, l16);
    }
  };

  // Per 64-k stage kt, two halves, each ending at a barrier:
  //   first half:  MFMAs on f0 (stage kt, k 0-31), reads of f1 (stage kt,
  //                k 32-63), loads of stage kt+2's first half into the buffer
  //                f0 came from (every wave read it before the last barrier);
  //   second half: MFMAs on f1, reads of f0 (stage kt+1, k 0-31), loads of
  //                stage kt+2's second half into the buffer f1 came from.
  // Loads are issued in a fixed order, 2 * LPL per half per lane, so "at most
  // 4 * LPL outstanding" at a barrier means everything issued more than two halves
  // ago has landed -- exactly the half the next half reads.  Past the last
  // stage the loads reload consumed stages into their own buffers and the
  // reads of "the next stage" read a buffer whose contents go unused (no
  // branches around either).
  const uint32_t nk = (R + DBK - 1) / DBK;
  // the epilogue's kernel arguments, loaded here rather than inside the loop,
  // where a pending scalar load would again force full LDS waits
  asm volatile("" ::"s"(C), "s"(Mo), "s"(No));
  Frags f0, f1;
  const uint32_t s1 = nk > 1 ? 1 : 0;
  issue_half(0, 0);
  issue_half(0, 1);
  issue_half(s1, 0);
  issue_half(s1, 1);
  // stage 0 in place (with a single stage, all loads; the repeat would
  // rewrite the buffers being read)
  if (nk > 1)
    __builtin_amdgcn_s_waitcnt(kWaitHalves);
  else
    __builtin_amdgcn_s_waitcnt(kWait0);
  __builtin_amdgcn_s_barrier();
  load_frags(hbuf(0, 0), f0);
  // every wave holds its f0 before the first half's loads overwrite that buffer
  __builtin_amdgcn_s_waitcnt(kWaitHalves);
  __builtin_amdgcn_s_barrier();
  for (uint32_t kt = 0; kt < nk; ++kt) {
    // stage kt+2 goes into stage kt's buffers; past the end, stage kt itself
    // is reloaded there (consumed, never read again)
    const uint32_t kn = kt + 2 < nk ? kt + 2 : kt;
    mma_read(f0, hbuf(kt, 1), f1, kn, 0);
    __builtin_amdgcn_s_waitcnt(kWaitHalves);
    __builtin_amdgcn_s_barrier();
    mma_read(f1, hbuf(kt + 1, 0), f0, kn, 1);
    __builtin_amdgcn_s_waitcnt(kWaitHalves);
    __builtin_amdgcn_s_barrier();
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  hazard_guard<7>(acc);

#pragma unroll
  for (int r = 0; r < TM; ++r)
#pragma unroll
    for (int c = 0; c < TN; ++c) {
      const uint32_t gc = n0 + wn * WTN + c * 16 + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t gr = m0 + wm * WT + r * 16 + 4 * kb + i;
        if (gr < Mo && gc < No) store_out(C + (size_t)gr * No + gc, acc[r][c][i]);
      }
    }
}

// f32 -> f16, round to nearest even (the cast of the output gradient)
__global__ void __launch_bounds__(256)
cast_f16_kernel(const float* __restrict__ src, uint16_t* __restrict__ dst, size_t n, bool vec) {
  const size_t stride = (size_t)gridDim.x * 256;
  if (vec) {   // 8 values per step, 16-byte aligned, n % 8 == 0
    for (size_t v = (size_t)blockIdx.x * 256 + threadIdx.x; v < n / 8; v += stride) {
      const float4 lo = reinterpret_cast<const float4*>(src)[2 * v];
      const float4 hi = reinterpret_cast<const float4*>(src)[2 * v + 1];
      const half8_t h = {(_Float16)lo.x, (_Float16)lo.y, (_Float16)lo.z, (_Float16)lo.w,
                         (_Float16)hi.x, (_Float16)hi.y, (_Float16)hi.z, (_Float16)hi.w};
      reinterpret_cast<uint4*>(dst)[v] = __builtin_bit_cast(uint4, h);
    }
  } else {
    for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < n; e += stride)
      dst[e] = __builtin_bit_cast(uint16_t, (_Float16)src[e]);
  }
}

__global__ void fill_zero_kernel(uint4* __restrict__ dst, size_t n16, uint8_t* __restrict__ tail, uint32_t ntail) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    dst[i] = uint4{0u, 0u, 0u, 0u};
  if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

}  // namespace

namespace {
#ifndef KAIO_GEMM_WN
#define KAIO_GEMM_WN 4
#endif
template <bool kATr, bool kBTr, typename OutT, bool kRagged>
hipError_t launch_dma(const uint16_t* a, uint32_t lda, const uint16_t* b, uint32_t ldb, OutT* c, uint32_t mo,
                      uint32_t no, uint32_t r, hipStream_t stream) {
  constexpr int WN = KAIO_GEMM_WN;
  const uint32_t mtiles = (mo + BM - 1) / BM, ntiles = (no + BN - 1) / BN;
  const size_t lds = (size_t)8 * HSLOTS * 16;
  auto* kern = &gemm_dma_kernel<kATr, kBTr, OutT, kRagged, WN>;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3(mtiles * ntiles), dim3(128 * WN), lds, stream, a, lda, b, ldb, c, mo, no, r,
                     mtiles, ntiles);
  return hipGetLastError();
}

// the direct-to-LDS kernel, whole 64-k stages only when the reduction allows
template <bool kATr, bool kBTr, typename OutT>
hipError_t launch_dma_any(const uint16_t* a, uint32_t lda, const uint16_t* b, uint32_t ldb, OutT* c, uint32_t mo,
                          uint32_t no, uint32_t r, hipStream_t stream) {
  return r % DBK == 0 ? launch_dma<kATr, kBTr, OutT, false>(a, lda, b, ldb, c, mo, no, r, stream)
                      : launch_dma<kATr, kBTr, OutT, true>(a, lda, b, ldb, c, mo, no, r, stream);
}
}  // namespace

namespace {
// The register-staged kernel.  An operand reads aligned 16-byte chunks when
// its stride and contiguous extent (the reduction for a reduction-contiguous
// operand, its index count for an index-contiguous one) are multiples of 8,
// clamped 16-byte chunks when that extent is at least 8, and elements
// otherwise (then both operands do, keeping the instantiations few).
template <int kAM, int kBM, bool kATr, bool kBTr, typename OutT>
void launch_reg_form(const uint16_t* a, uint32_t lda, const uint16_t* b, uint32_t ldb, OutT* c, uint32_t mo,
                     uint32_t no, uint32_t r, uint32_t mtiles, uint32_t ntiles, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_reg_kernel<kAM, kBM, kATr, kBTr, OutT>), dim3(mtiles * ntiles), dim3(THREADS), 0,
                     stream, a, lda, b, ldb, c, mo, no, r, mtiles);
}
template <bool kATr, bool kBTr, typename OutT>
hipError_t launch_reg(const uint16_t* a, uint32_t lda, const uint16_t* b, uint32_t ldb, OutT* c, uint32_t mo,
                      uint32_t no, uint32_t r, hipStream_t stream) {
  const uint32_t mtiles = (mo + BM - 1) / BM, ntiles = (no + BN - 1) / BN;
  const uint32_t a_ext = kATr ? mo : r, b_ext = kBTr ? no : r;
  const int a_mode = lda % 8 == 0 && a_ext % 8 == 0 ? kLoadAligned : (a_ext >= 8 ? kLoadClamped : kLoadElement);
  const int b_mode = ldb % 8 == 0 && b_ext % 8 == 0 ? kLoadAligned : (b_ext >= 8 ? kLoadClamped : kLoadElement);
  if (a_mode == kLoadElement || b_mode == kLoadElement)
    launch_reg_form<kLoadElement, kLoadElement, kATr, kBTr>(a, lda, b, ldb, c, mo, no, r, mtiles, ntiles, stream);
  else if (a_mode == kLoadAligned && b_mode == kLoadAligned)
    launch_reg_form<kLoadAligned, kLoadAligned, kATr, kBTr>(a, lda, b, ldb, c, mo, no, r, mtiles, ntiles, stream);
  else if (a_mode == kLoadAligned)
    launch_reg_form<kLoadAligned, kLoadClamped, kATr, kBTr>(a, lda, b, ldb, c, mo, no, r, mtiles, ntiles, stream);
  else if (b_mode == kLoadAligned)
    launch_reg_form<kLoadClamped, kLoadAligned, kATr, kBTr>(a, lda, b, ldb, c, mo, no, r, mtiles, ntiles, stream);
  else
    launch_reg_form<kLoadClamped, kLoadClamped, kATr, kBTr>(a, lda, b, ldb, c, mo, no, r, mtiles, ntiles, stream);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm_f16f32(const uint16_t* a, const uint16_t* b, float* c,
                              uint32_t m, uint32_t n, uint32_t k, hipStream_t stream) {
  // Direct-to-LDS path: A's 16-byte reduction chunks need k % 8 == 0 (a chunk
  // never straddles the end of the reduction), B's index chunks n % 8 == 0;
  // 32-bit per-lane byte offsets need 256 * k * 2 and 64 * n * 2 below 2^31.
  if (k > 0 && k % 8 == 0 && n % 8 == 0 && k < (1u << 22) && n < (1u << 24))
    return launch_dma_any<false, true, float>(a, k, b, n, c, m, n, k, stream);
  return launch_reg<false, true, float>(a, k, b, n, c, m, n, k, stream);
}

hipError_t launch_gemm_f16f32_bwd(const uint16_t* a, const uint16_t* b, const float* grad, uint16_t* grad_a,
                                  uint16_t* grad_b, uint16_t* grad16, uint32_t m, uint32_t n, uint32_t k,
                                  hipStream_t stream) {
  // grad16 = f16(grad), [m, n]
  const size_t mn = (size_t)m * n;
  const bool vec = mn % 8 == 0 && (uintptr_t)grad % 16 == 0 && (uintptr_t)grad16 % 16 == 0;
  size_t blocks = ((vec ? mn / 8 : mn) + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(cast_f16_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, grad, grad16, mn, vec);
  if (hipError_t e = hipGetLastError()) return e;
  // grad_a[m, k] = grad16[m, n] . b[k, n]^T: both operands reduction (n)
  // contiguous, so n % 8 == 0 (no 16-byte chunk straddles the end of a row)
  hipError_t e;
  if (n % 8 == 0 && n < (1u << 22))
    e = launch_dma_any<false, false, uint16_t>(grad16, n, b, n, grad_a, m, k, n, stream);
  else
    e = launch_reg<false, false, uint16_t>(grad16, n, b, n, grad_a, m, k, n, stream);
  if (e != hipSuccess) return e;
  // grad_b[k, n] = a[m, k]^T . grad16[m, n]: both operands index contiguous;
  // any m (whole reduction rows past m read as zeros)
  if (k % 8 == 0 && n % 8 == 0 && k < (1u << 24) && n < (1u << 24))
    e = launch_dma_any<true, true, uint16_t>(a, k, grad16, n, grad_b, k, n, m, stream);
  else
    e = launch_reg<true, true, uint16_t>(a, k, grad16, n, grad_b, k, n, m, stream);
  return e;
}

// ---------------------------------------------------------------------------
// Allocation-free backward: f16(grad) staged in a static device buffer.
//
// `scratch` is a file-scope device array: every device that loads this code
// object holds its own copy, at its own address, until the process ends.  In
// host code its name is only a host-side stand-in, so the kernels are given
// the device address hipGetSymbolAddress returns, looked up once per device
// (with that device current) and kept.  Calls that overlap in time on one
// device share the array and race; nothing in it has to start at zero (the
// cast overwrites the m*n halves the two products read).
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint16_t scratch[kGemmBwdScratchBytes / 2];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
uint16_t* g_scratch_ptr[kMaxScratchDevices] = {};

hipError_t scratch_of_current_device(uint16_t** out) {
  int dev = -1;
  if (hipError_t e = hipGetDevice(&dev)) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = static_cast<uint16_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

hipError_t launch_gemm_f16f32_bwd_noalloc(const uint16_t* a, const uint16_t* b, const float* grad,
                                          uint16_t* grad_a, uint16_t* grad_b, uint32_t m, uint32_t n,
                                          uint32_t k, hipStream_t stream) {
  if ((uint64_t)m * n * 2 > kGemmBwdScratchBytes) return hipErrorInvalidValue;   // checked by the caller
  uint16_t* g16 = nullptr;
  if (hipError_t e = scratch_of_current_device(&g16)) return e;
  return launch_gemm_f16f32_bwd(a, b, grad, grad_a, grad_b, g16, m, n, k, stream);
}

hipError_t launch_fill_zero(void* dst, size_t bytes, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  const uint32_t ntail = (uint32_t)(bytes % 16);
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream,
                     reinterpret_cast<uint4*>(dst), n16, reinterpret_cast<uint8_t*>(dst) + n16 * 16, ntail);
  return hipGetLastError();
}

}  // namespace kaio
