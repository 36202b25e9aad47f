// W4A16 fused tri-output QKV projection -- split-K kernel for small m (m <= 64).
//
// Operation: kaio-candle 0.2.0, src/qkv_project_int4.rs (module doc and the
// doc comment of qkv_project_int4); same contract as the tile kernel.
//
// gfx950 design
// -------------
// At small m the 4-bit weights are almost all of the bytes: every weight must
// stream from HBM once, spread over the whole chip, so the reduction axis is
// split across the waves of a workgroup (the tile kernel's column tiles would
// leave most CUs idle).  The arithmetic intensity (~31 flop/byte at m = 8) is
// above the f32 VALU ridge, so the products still run on MFMA: x is the A
// operand in RT row tiles of 16 (rows past m repeat row m-1), the weights the
// B operand.
// * Workgroup = WAVES waves on a strip of 16*VEC columns of ONE output.  Lane
//   (kb, c) loads one VEC-word vector = the words of columns VEC*c .. VEC*c+VEC-1
//   at packed row kb of a 32-k step: each word is the B operand of VEC x RT
//   MFMAs (one per row tile), whose column c stands for output column
//   VEC*c + t.  A wave-wide load covers 4 packed rows x 64*VEC contiguous bytes.
// * Every workgroup reads the same small x.  Each wave loads its groups' x
//   rows as 256-byte row segments (4 rows per load) into a wave-private LDS
//   slice and reads its A fragments back from there; fragment-shaped loads
//   (16 rows, 64 bytes each, per load) cost ~1.5 us more per call at
//   m = 8, n = k = 4096.
// * Split-K across the waves (wave w takes groups [wG/W, (w+1)G/W)); each
//   wave streams its groups GCHUNK at a time through two register buffers,
//   the next chunk's loads in flight while the current chunk computes, or,
//   from 40 to 64 groups at m <= 8, issues all of its groups' loads at once
//   with x in LDS by direct loads.  No load sits under a branch (see the main
//   loop); a partial last strip loads clamped columns (see the body).
// * INT4 unpack once per word whatever RT is: with one row tile, in
//   nibble-interleaved k order (9 VALU ops per word) with the x fragments
//   permuted to the same order in registers; with two or more, in k order
//   (10 ops per word, values q * 2^-9, the factor returned through the scale)
//   with no permutation.
// * Per group: 4 chained MFMAs per (column set, row tile) into a fresh
//   partial, then acc += partial * scale in f32 (every product exact, as in
//   the tile kernel).
// * The wave partial sums meet in LDS and are added in a fixed order, so
//   results are deterministic; then f32 -> f16 (RNE) and row stores.
// Configurations (row tiles per wave x row blocks, columns per strip, waves)
// are chosen per m so that the register file holds two chunks plus the
// accumulators without spilling and the reduction buffer stays at 64 KiB
// (plus 68 KiB of x slices): m <= 16: 1 x 1, 64, 16 (8 x rows kept when
// m <= 8); m <= 32: 2 x 1, 64, 8; m <= 64: 2 x 2, 64, 8.  Larger m (and INT4
// from m = 33 when the group count divides by 4) runs the tile kernel, which
// unpacks each word once per tile of 64, 96 or 128 rows.

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

#ifndef KAIO_DECODE_GCHUNK
#define KAIO_DECODE_GCHUNK 1
#endif

namespace kaio {
namespace {

constexpr int GCHUNK = KAIO_DECODE_GCHUNK;    // groups loaded per pass of a wave

template <int V> struct WordVec;
template <> struct WordVec<1> { using T = uint32_t; };
template <> struct WordVec<2> { using T = u32x2; };
template <> struct WordVec<4> { using T = u32x4; };

// Loads.  In the 16-wave configurations (straight-line, two groups per wave)
// every load is a buffer load: a wave-uniform base (a descriptor in SGPRs)
// plus one 32-bit per-lane byte offset fixed for the whole kernel, instead of
// a 64-bit per-lane address -- fewer VGPRs and no 64-bit address VALU (m = 8:
// 108 -> 100 VGPRs, 7.47 -> 7.20 us; W8A16 fits 16 waves without spilling).
// The 8-wave configurations loop over their groups, and rebuilding
// descriptors there cost 12-20%: they keep global loads.  Buffer offsets stay
// below 2^32 by the host-side limits (k < 2^24, n < 2^26, m <= 64): x rows
// <= 63 of 2k bytes; weights < 8 packed rows of 4n bytes.
// Packed weights that one wave alone reads (rows not split across waves) carry
// the non-temporal hint: they stream past the caches instead of displacing the
// small x that every workgroup re-reads (n = k = 4096: m = 8 7.94 -> 7.37 us,
// m = 16 8.94 -> 8.25, m = 32 12.37 -> 11.76).  When RSPLIT waves read the
// same words (m > 32) the hint would defeat that reuse (+6% with the rows
// split four ways), and
// the scales are faster without it.
template <bool kOnce, typename T>
__device__ __forceinline__ T load_w(const T* p) {
  if constexpr (kOnce) return __builtin_nontemporal_load(p);
  else return *p;
}
constexpr int kBufferFlags = 0x00020000;   // raw buffer, 32-bit data format
// records = -1: no range limit (every offset is in bounds by construction);
// 0: every load through the descriptor is out of range -- it returns zeros
// without touching memory (still one load for the wait counts).
// records must be the same in every lane of the wave (every caller's choice
// depends on the wave's group range only).  It is read from the first lane so
// that the compiler keeps the descriptor in scalar registers: a range it
// computes with a vector select makes it wrap each load in a loop over the
// lanes' distinct descriptors.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* base, int records = -1) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, __builtin_amdgcn_readfirstlane(records),
                                           kBufferFlags);
}
template <int V, int kPolicy>
__device__ __forceinline__ typename WordVec<V>::T buf_words(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (V == 4) return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kPolicy);
  else if constexpr (V == 2) return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kPolicy);
  else return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kPolicy);
}
template <int V> struct HalfVec { typedef uint16_t T __attribute__((ext_vector_type(V))); };
template <> struct HalfVec<1> { typedef uint16_t T; };
template <int V>
__device__ __forceinline__ typename HalfVec<V>::T buf_halves(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  using HV = typename HalfVec<V>::T;
  if constexpr (V == 4) return __builtin_bit_cast(HV, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
  else if constexpr (V == 2) return __builtin_bit_cast(HV, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
  else return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

// kFull: n % BN == 0, so every strip is complete and the vector loads of
// weights (VEC words) and scales (VEC halves) stay inside their rows.
// RSPLIT > 1 splits the rows across waves as well: wave w takes row block
// w % RSPLIT (16*RT rows) and reduction part w / RSPLIT of WAVES / RSPLIT.
// XR = rows of x a wave keeps per group (a multiple of 4, at most 16*RT;
// 8 when m <= 8, which leaves registers for two groups in flight).
// BITS = 4 (W4A16: one packed word per 8 k of a column) or 8 (W8A16: two).
// kTrim: some wave's group range is not exactly two chunks (its loop runs
// past the range), and the weight loads past it go through a zero-range
// descriptor (16-wave buffer-load configurations, n % 4 == 0).
// NG > 0: every wave issues the loads of all its groups (at most NG) at once
// and x goes to LDS by direct loads, which frees the registers that holding
// x would take (16 waves, n % 4 == 0, m <= 8, at most NG groups per wave).
template <int BITS, int RT, int RSPLIT, int VEC, int WAVES, bool kFull, int XR, bool kTrim = false, int NG = 0>
__global__ void __launch_bounds__(WAVES * 64, 1)
qkv_decode_kernel(QkvProblem p, uint32_t nstrips) {
  constexpr int THREADS = WAVES * kWave;
  constexpr int WPK = BITS / 4;                 // packed words per 8 k of a column
  constexpr int PR = 16 * WPK;                  // packed rows per group of 128 k
  constexpr int BN = 16 * VEC;                  // columns per strip
  constexpr int KSPLIT = WAVES / RSPLIT;        // waves per row block, splitting the reduction
  constexpr int ROWS = 16 * RT * RSPLIT;        // rows per workgroup
  static_assert(VEC == 1 || VEC == 2 || VEC == 4, "vector width");
  static_assert(KSPLIT * RSPLIT == WAVES, "row split must divide the waves");
  static_assert(KSPLIT * ROWS * BN * 4 <= 65536, "reduction buffer");
  using WV = typename WordVec<VEC>::T;
  constexpr int XROWS = XR;                     // x rows of a wave's row block kept in LDS
  // Weights in k order (q * 2^-9, 10 VALU ops per word, x fragments used as
  // read) when every word feeds two or more row tiles; otherwise in the
  // nibble-interleaved order (9 ops per word) with each x fragment permuted
  // to match (4 ops), which costs less when a word feeds one row tile.
  constexpr bool kNatural = RT >= 2 || BITS == 8;
  static_assert(XR % 4 == 0 && XR <= 16 * RT, "x rows per wave");
  constexpr int XLD = kGroup / 8 + 1;           // 16-byte chunks per padded LDS row of x
  static_assert(NG == 0 || (WAVES == 16 && RT == 1 && XR == 8 && BITS == 4 && NG <= 4),
                "all groups in flight: the 16-wave m <= 8 configuration only");
  // LDS: the reduction buffer, and per wave either one padded x slice (x
  // staged through registers) or NG unpadded, swizzled ones (direct loads;
  // the reduction buffer then reuses them, once every wave is done with x)
  using RedT = float[KSPLIT][ROWS][BN];
  RedT* red_p;
  uint4* xl_base;
  if constexpr (NG == 0) {
    __shared__ float red_s[KSPLIT][ROWS][BN];
    __shared__ uint4 xl[WAVES][XROWS * XLD];
    red_p = &red_s;
    xl_base = &xl[0][0];
  } else {
    static_assert(KSPLIT * ROWS * BN * 4 <= WAVES * NG * XROWS * 16 * 16, "reduction buffer fits the x slices");
    __shared__ uint4 xd[WAVES * NG * XROWS * 16];
    red_p = reinterpret_cast<RedT*>(xd);
    xl_base = xd;
  }
  RedT& red = *red_p;

  // The body.  kF: whole-vector loads of each lane's VEC columns (16-byte
  // weights, 8-byte scales; aligned when n % 4 == 0).  kG: the strip's last
  // columns may lie past N: stores are guarded, and with kF a lane whose
  // columns lie past N (with n % 4 == 0 all four do, or none) loads the last
  // VEC columns instead -- valid memory; MFMA columns do not mix and those
  // outputs are never stored.  Without kF, every column load is guarded.  A
  // kernel built for n % BN != 0 thus runs whole-vector loads on every strip
  // when n % 4 == 0, and the column-guarded loads only otherwise.
  auto body = [&](auto full_tag, auto guard_tag) {
    constexpr bool kF = decltype(full_tag)::value;
    constexpr bool kG = decltype(guard_tag)::value;
    static_assert(kF || kG, "guarded loads go with guarded stores");
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t kb = lane >> 4;
    const uint32_t l16 = lane & 15;

    const uint32_t q = blockIdx.x / nstrips;
    const uint32_t n0 = (blockIdx.x % nstrips) * BN;
    const uint32_t M = p.m, N = p.n, K = p.k;
    const uint32_t G = K / kGroup;
    const uint32_t rblk = wave % RSPLIT, kpart = wave / RSPLIT;
    const uint32_t g_begin = (uint32_t)(((uint64_t)kpart * G) / KSPLIT);
    const uint32_t g_end = (uint32_t)(((uint64_t)(kpart + 1) * G) / KSPLIT);

    const uint32_t* w = q == 0 ? p.w[0] : (q == 1 ? p.w[1] : p.w[2]);
    const uint16_t* s = q == 0 ? p.s[0] : (q == 1 ? p.s[1] : p.s[2]);
    const uint32_t colv = n0 + VEC * l16;     // first of the lane's VEC columns
    const uint32_t colv_ld = kF && kG && colv >= N ? N - VEC : colv;   // the columns it loads
    // without kF, column by column: columns past N load column N-1 instead
    // (no load sits under a branch, which would make the compiler's waits
    // conservative; those outputs are never stored)
    auto col_of = [&](int t) { return colv + t < N ? colv + t : N - 1; };
    // x of a group reaches the MFMAs through a wave-private LDS slice: load j
    // brings rows 4j .. 4j+3 of the wave's row block, 256 contiguous bytes each
    // (lane l: row 4j + l/16, 16-byte chunk l % 16), and each A fragment is read
    // back from there.  Loading the fragments straight from memory would make
    // every load touch 16 rows 2*K bytes apart with 64 bytes each, and the
    // whole chip reads this same x: that costs ~1.5 us per call at m = 8,
    // n = k = 4096.  Rows are padded to 17 chunks, so a fragment read (16 rows,
    // one chunk each) is free of bank conflicts.
    // Rows past M repeat row M-1 (their outputs are never stored, and MFMA rows
    // do not mix).  Every load is issued, whatever M (repeated rows read the same
    // addresses): a load under a branch would make the compiler wait for all
    // loads in flight, the next group's included, before the first LDS write.
    const uint32_t xbase = 16 * RT * rblk;
    const uint32_t xvalid = M > xbase ? (M - xbase < (uint32_t)XROWS ? M - xbase : XROWS) : 1;  // rows kept
    // element offset of load j's chunk within a group's x columns (computed at
    // each load: few registers are free in the widest configuration)
    auto xoff = [&](int j) {
      const uint32_t lr = 4 * j + kb;
      const uint32_t row = xbase + (lr < xvalid ? lr : xvalid - 1);
      return (row < M ? row : M - 1) * K + l16 * 8;
    };
    uint32_t xfrag[RT];       // LDS row of the lane's A fragment in row tile r
  #pragma unroll
    for (int r = 0; r < RT; ++r) {
      const uint32_t lr = 16 * r + l16;
      xfrag[r] = (lr < xvalid ? lr : xvalid - 1) * XLD + kb;
    }
    uint4* const xw = xl_base + wave * (NG == 0 ? XROWS * XLD : NG * XROWS * 16);
    // lane (kb, c) of k-step ks holds packed rows WPK*(4ks + kb) + j, j < WPK:
    // the 8 consecutive k of its B operand.  Byte offset from the row
    // PR*g + 4*WPK*ks + j of the load's base:
    const uint32_t woff = ((WPK * kb) * N + colv_ld) * 4;
    const uint32_t* wlane = w + (size_t)(WPK * kb) * N + colv_ld;   // the same, as an address
    constexpr int kWPolicy = RSPLIT == 1 ? 2 : 0;   // non-temporal when one wave reads each word
    constexpr bool kBuf = WAVES == 16;              // buffer loads (see above)
    using ScT = std::conditional_t<kBuf, uint16_t, uint32_t>;

    floatx4 acc[VEC][RT];
  #pragma unroll
    for (int t = 0; t < VEC; ++t)
  #pragma unroll
      for (int r = 0; r < RT; ++r) acc[t][r] = floatx4{0.f, 0.f, 0.f, 0.f};

    struct Chunk {
      uint32_t wv[GCHUNK][4][WPK][VEC];
      uint4 xs[GCHUNK][XROWS / 4];     // x rows 4j .. 4j+3 of the group, 16 bytes per lane
      // f16 bits of the scales: packed two per register in the 16-wave
      // configurations (register budget), one per register otherwise (1-2% faster there)
      ScT sc[GCHUNK][VEC];
    };
    // Loads of GCHUNK groups starting at g0.  Groups past the wave's range are
    // clamped to its last group (loaded, never used) so that every chunk issues
    // the same loads and the compiler can keep the next chunk in flight.  With
    // kTrim, the weight loads of such a group go through a zero-range
    // descriptor instead: a repeat of streamed (non-temporal) words was often
    // fetched from memory again (n = 4096, k = 8192, m = 8: 1.17x the
    // algorithmic bytes).
    auto load_chunk = [&](uint32_t g0, Chunk& c, bool checked) {
  #pragma unroll
      for (int gi = 0; gi < GCHUNK; ++gi) {
        const bool live = !checked || g0 + gi < g_end;   // checked = false: inside the range
        const uint32_t g = live ? g0 + gi : g_end - 1;
        // x first: loads complete in issue order, so the LDS copy of x (needed
        // before any MFMA) need not wait for the weights of later k-steps
        if constexpr (kBuf) {
          const __amdgpu_buffer_rsrc_t xr = rsrc_of(p.x + (size_t)g * kGroup);
  #pragma unroll
          for (int j = 0; j < XROWS / 4; ++j)
            c.xs[gi][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, xoff(j) * 2, 0, 0));
  #pragma unroll
          for (int ks = 0; ks < 4; ++ks)
  #pragma unroll
            for (int j = 0; j < WPK; ++j) {
              const __amdgpu_buffer_rsrc_t wr =
                  rsrc_of(w + ((size_t)g * PR + ks * 4 * WPK + j) * N, kTrim && kF && !live ? 0 : -1);
              if (kF) {
                const WV v = buf_words<VEC, kWPolicy>(wr, woff);
                __builtin_memcpy(c.wv[gi][ks][j], &v, sizeof(v));
              } else {
  #pragma unroll
                for (int t = 0; t < VEC; ++t)
                  c.wv[gi][ks][j][t] = buf_words<1, kWPolicy>(wr, ((WPK * kb) * N + col_of(t)) * 4);
              }
            }
          const __amdgpu_buffer_rsrc_t sr = rsrc_of(s + (size_t)g * N);
          if (kF) {
            const auto sv = buf_halves<VEC>(sr, colv_ld * 2);
            __builtin_memcpy(c.sc[gi], &sv, sizeof(sv));
          } else {
  #pragma unroll
            for (int t = 0; t < VEC; ++t) c.sc[gi][t] = buf_halves<1>(sr, col_of(t) * 2);
          }
        } else {
  #pragma unroll
          for (int j = 0; j < XROWS / 4; ++j)
            c.xs[gi][j] = *reinterpret_cast<const uint4*>(p.x + xoff(j) + (size_t)g * kGroup);
  #pragma unroll
          for (int ks = 0; ks < 4; ++ks)
  #pragma unroll
            for (int j = 0; j < WPK; ++j) {
              const size_t roff = ((size_t)g * PR + ks * 4 * WPK + j) * N;
              if (kF) {
                const WV v = load_w<RSPLIT == 1>(reinterpret_cast<const WV*>(wlane + roff));
                __builtin_memcpy(c.wv[gi][ks][j], &v, sizeof(v));
              } else {
  #pragma unroll
                for (int t = 0; t < VEC; ++t)
                  c.wv[gi][ks][j][t] = load_w<RSPLIT == 1>(w + (size_t)(WPK * kb) * N + roff + col_of(t));
              }
            }
          if (kF) {
            using HV = typename HalfVec<VEC>::T;
            const HV sv = *reinterpret_cast<const HV*>(s + (size_t)g * N + colv_ld);
            uint16_t sh[VEC];
            __builtin_memcpy(sh, &sv, sizeof(sv));
  #pragma unroll
            for (int t = 0; t < VEC; ++t) c.sc[gi][t] = sh[t];
          } else {
  #pragma unroll
            for (int t = 0; t < VEC; ++t) c.sc[gi][t] = s[(size_t)g * N + col_of(t)];
          }
        }
      }
    };
    auto compute_chunk = [&](uint32_t g0, const Chunk& c, bool checked) {
  #pragma unroll
      for (int gi = 0; gi < GCHUNK; ++gi) {
        if (!checked || g0 + gi < g_end) {   // wave-uniform
          // LDS accesses of one wave execute in order: these writes follow the
          // previous group's fragment reads, and the reads below follow them;
          // the empty asm statements keep the compiler from reordering them.
          asm volatile("" ::: "memory");
  #pragma unroll
          for (int j = 0; j < XROWS / 4; ++j) xw[(4 * j + kb) * XLD + l16] = c.xs[gi][j];
          asm volatile("" ::: "memory");
          floatx4 part[VEC][RT];
  #pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            half8_t a[RT];
  #pragma unroll
            for (int r = 0; r < RT; ++r)
              a[r] = kNatural ? __builtin_bit_cast(half8_t, xw[xfrag[r] + 4 * ks])
                              : permute_x_like_int4x8(xw[xfrag[r] + 4 * ks]);
  #pragma unroll
            for (int t = 0; t < VEC; ++t) {
              half8_t b;
              if constexpr (kNatural) {
                uint32_t words[WPK];
  #pragma unroll
                for (int j = 0; j < WPK; ++j) words[j] = c.wv[gi][ks][j][t];
                b = unpack_b_scaled<BITS>(words);
              } else {
                b = unpack_int4x8_interleaved(c.wv[gi][ks][0][t]);
              }
  #pragma unroll
              for (int r = 0; r < RT; ++r)
                part[t][r] = mfma16x16x32(a[r], b, ks == 0 ? floatx4{0.f, 0.f, 0.f, 0.f} : part[t][r]);
            }
          }
  #pragma unroll
          for (int t = 0; t < VEC; ++t) {
            const float sf = kNatural ? h2f((uint16_t)c.sc[gi][t]) * kUnpackScaledInv : h2f((uint16_t)c.sc[gi][t]);
  #pragma unroll
            for (int r = 0; r < RT; ++r)
  #pragma unroll
              for (int i = 0; i < 4; ++i) acc[t][r][i] = __builtin_fmaf(part[t][r][i], sf, acc[t][r][i]);
          }
        }
      }
    };

    if constexpr (NG > 0) {
      // Every group of the wave in flight at once: first the x of every group,
      // two direct loads each (rows 4j .. 4j+3, 16 chunks each, into slice gi;
      // the chunk of row r at position c sits at c ^ r, so that a fragment read
      // of 8 rows hits 8 distinct 16-byte bank groups), then per group four
      // weight loads and one scale load.  x goes first because the compiler
      // makes the first read of any slice wait for every direct load issued
      // before it (it cannot tell the slices apart), so x issued per group
      // would hold group 0's compute until later groups' x had landed.  Groups
      // past the wave's range load through zero-range descriptors.
      struct WChunk {
        uint32_t wv[4][VEC];
        uint16_t sc[VEC];
      };
      WChunk c[NG];
  #pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        const bool live = g_begin + gi < g_end;
        const uint32_t g = live ? g_begin + gi : g_begin;
        const __amdgpu_buffer_rsrc_t xr = rsrc_of(p.x + (size_t)g * kGroup, live ? -1 : 0);
  #pragma unroll
        for (int j = 0; j < XROWS / 4; ++j) {
          const uint32_t lr = 4 * j + kb;                 // LDS row of this lane's chunk
          const uint32_t row = xbase + (lr < xvalid ? lr : xvalid - 1);
          const uint32_t off = ((row < M ? row : M - 1) * K + (l16 ^ lr) * 8) * 2;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              xr, (__attribute__((address_space(3))) void*)(xw + (gi * XROWS + 4 * j) * 16), 16, off, 0, 0, 0);
        }
      }
      // the load order the waits below count on: all x, then the weights and scales group by group
      asm volatile("" ::: "memory");
  #pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        const bool live = g_begin + gi < g_end;
        const uint32_t g = live ? g_begin + gi : g_begin;
  #pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const __amdgpu_buffer_rsrc_t wr = rsrc_of(w + ((size_t)g * PR + ks * 4) * N, live ? -1 : 0);
          const WV v = buf_words<VEC, kWPolicy>(wr, woff);
          __builtin_memcpy(c[gi].wv[ks], &v, sizeof(v));
        }
        const auto sv = buf_halves<VEC>(rsrc_of(s + (size_t)g * N), colv_ld * 2);
        __builtin_memcpy(c[gi].sc, &sv, sizeof(sv));
        asm volatile("" ::: "memory");
      }
      const uint32_t frow = l16 < xvalid ? l16 : xvalid - 1;   // the lane's A row (rows past m repeat)
  #pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        if (g_begin + gi < g_end) {   // wave-uniform
          // every x has landed, and group gi's weights and scales, once at most
          // the later groups' 5 loads each are outstanding; loads complete in
          // issue order
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(5 * (NG - 1 - gi)) : "memory");
          floatx4 part[VEC];
  #pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const uint32_t ch = 4 * ks + kb;
            const half8_t a = permute_x_like_int4x8(xw[(gi * XROWS + frow) * 16 + (ch ^ frow)]);
  #pragma unroll
            for (int t = 0; t < VEC; ++t) {
              const half8_t b = unpack_int4x8_interleaved(c[gi].wv[ks][t]);
              part[t] = mfma16x16x32(a, b, ks == 0 ? floatx4{0.f, 0.f, 0.f, 0.f} : part[t]);
            }
          }
  #pragma unroll
          for (int t = 0; t < VEC; ++t) {
            const float sf = h2f(c[gi].sc[t]);
  #pragma unroll
            for (int i = 0; i < 4; ++i) acc[t][0][i] = __builtin_fmaf(part[t][i], sf, acc[t][0][i]);
          }
        }
      }
      __syncthreads();   // every wave is done with its x slices before the reduction reuses them
    } else if (g_begin < g_end) {
      // two register buffers used ping-pong: chunk c+1 is in flight while
      // chunk c computes.  Every load is issued unconditionally (past the
      // wave's range they repeat its last group, which the cache holds): a load
      // under a branch leaves the compiler's wait counts conservative where the
      // paths meet, and it would wait for chunk c+1 before computing chunk c.
      Chunk ca, cb;
      if (g_end - g_begin == 2 * GCHUNK) {
        // exactly two chunks (every wave at m <= 16, k = 4096): straight-line
        load_chunk(g_begin, ca, false);
        load_chunk(g_begin + GCHUNK, cb, false);
        compute_chunk(g_begin, ca, false);
        compute_chunk(g_begin + GCHUNK, cb, false);
      } else {
        load_chunk(g_begin, ca, true);
        load_chunk(g_begin + GCHUNK, cb, true);
        for (uint32_t g0 = g_begin; g0 < g_end; g0 += 2 * GCHUNK) {
          compute_chunk(g0, ca, true);
          load_chunk(g0 + 2 * GCHUNK, ca, true);
          compute_chunk(g0 + GCHUNK, cb, true);
          load_chunk(g0 + 3 * GCHUNK, cb, true);
        }
      }
    }

    // lane holds rows 16r + 4*kb + i of its row block, MFMA column l16 = output column VEC*l16 + t
  #pragma unroll
    for (int t = 0; t < VEC; ++t)
  #pragma unroll
      for (int r = 0; r < RT; ++r)
  #pragma unroll
        for (int i = 0; i < 4; ++i)
          red[kpart][16 * RT * rblk + 16 * r + 4 * kb + i][VEC * l16 + t] = acc[t][r][i];
    __syncthreads();

    uint16_t* __restrict__ out = q == 0 ? p.out[0] : (q == 1 ? p.out[1] : p.out[2]);
    for (uint32_t e = tid; e < M * BN; e += THREADS) {
      const uint32_t row = e / BN, c = e % BN;
      float sum = 0.f;
  #pragma unroll
      for (int kp = 0; kp < KSPLIT; ++kp) sum += red[kp][row][c];
      const uint32_t gc = n0 + c;
      if (!kG || gc < N) out[(size_t)row * N + gc] = __builtin_bit_cast(uint16_t, (_Float16)sum);
    }
  };
  // Kernels with trimmed loads or all groups in flight are launched for n % 4 == 0 only and
  // do not build the column-by-column body.
  if constexpr (kFull) {
    body(std::true_type{}, std::false_type{});
  } else {
    bool done = false;
    if constexpr (NG == 0 && !kTrim) {
      if (p.n % 4 != 0) {
        body(std::false_type{}, std::true_type{});
        done = true;
      }
    }
    if (!done) {
      if ((blockIdx.x % nstrips + 1) * BN <= p.n)
        body(std::true_type{}, std::false_type{});
      else
        body(std::true_type{}, std::true_type{});
    }
  }
}

// kOnlyFull: the caller guarantees n % BN == 0 (only the full-strip kernel is built)
template <int BITS, int RT, int RSPLIT, int VEC, int WAVES, int XR = 16 * RT, bool kOnlyFull = false>
hipError_t launch_split_k(const QkvProblem& p, hipStream_t stream) {
  constexpr uint32_t BN = 16 * VEC;
  const uint32_t nstrips = (p.n + BN - 1) / BN;
  const dim3 grid(3 * nstrips), block(WAVES * kWave);
  // every wave with exactly two chunks (k = 4096 at 16 waves): the straight-line path only
  constexpr uint32_t KSPLIT = WAVES / RSPLIT;
  const bool straight = p.k / kGroup == 2 * GCHUNK * KSPLIT;
  if constexpr (WAVES == 16) {
    if ((kOnlyFull || p.n % BN == 0) && !straight) {
      hipLaunchKernelGGL((qkv_decode_kernel<BITS, RT, RSPLIT, VEC, WAVES, true, XR, true>), grid, block, 0, stream,
                         p, nstrips);
      return hipGetLastError();
    }
    if constexpr (!kOnlyFull) {
      if (p.n % 4 == 0 && !straight) {
        hipLaunchKernelGGL((qkv_decode_kernel<BITS, RT, RSPLIT, VEC, WAVES, false, XR, true>), grid, block, 0,
                           stream, p, nstrips);
        return hipGetLastError();
      }
    }
  }
  if (kOnlyFull || p.n % BN == 0)
    hipLaunchKernelGGL((qkv_decode_kernel<BITS, RT, RSPLIT, VEC, WAVES, true, XR>), grid, block, 0, stream, p,
                       nstrips);
  else if constexpr (!kOnlyFull)
    hipLaunchKernelGGL((qkv_decode_kernel<BITS, RT, RSPLIT, VEC, WAVES, false, XR>), grid, block, 0, stream, p,
                       nstrips);
  return hipGetLastError();
}

// m <= 8, n % 4 == 0, 16 waves owning 3 or 4 groups each: all of a wave's
// groups in flight, x through direct LDS loads
template <int NG>
hipError_t launch_all_groups(const QkvProblem& p, hipStream_t stream) {
  const uint32_t nstrips = (p.n + 63) / 64;
  if (p.n % 64 == 0)
    hipLaunchKernelGGL((qkv_decode_kernel<4, 1, 1, 4, 16, true, 8, false, NG>), dim3(3 * nstrips),
                       dim3(16 * kWave), 0, stream, p, nstrips);
  else
    hipLaunchKernelGGL((qkv_decode_kernel<4, 1, 1, 4, 16, false, 8, false, NG>), dim3(3 * nstrips),
                       dim3(16 * kWave), 0, stream, p, nstrips);
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_decode_bits(const QkvProblem& p, hipStream_t stream) {
  if constexpr (BITS == 4) {
    // It pays once the 16 waves own 2.5 groups or more on average (m = 8,
    // n = 4096: k = 5120 11.9 -> 11.1 us, 6144 12.7 -> 11.6, 8192 15.1 ->
    // 14.7); from 33 to 39 groups most waves own two and it gains nothing.
    const uint32_t groups = p.k / kGroup;
    if (p.m <= 8 && p.n % 4 == 0 && groups >= 40 && groups <= 64)
      return groups <= 48 ? launch_all_groups<3>(p, stream) : launch_all_groups<4>(p, stream);
  }
  // INT8 words are twice the registers per group: 16-wave workgroups fit
  // (128 VGPRs, buffer loads) only with full strips at m <= 8; otherwise INT8
  // keeps the 8-wave register budget (each wave then streams four groups).
  // m = 8, n = k = 4096: 12.66 us at 8 waves, 11.57 at 16.
  if (BITS == 8 && p.m <= 8 && p.n % 64 == 0) return launch_split_k<BITS, 1, 1, 4, 16, 8, true>(p, stream);
  constexpr int kSmallWaves = BITS == 8 ? 8 : 16;
  if (p.m <= 8) return launch_split_k<BITS, 1, 1, 4, kSmallWaves, 8>(p, stream);
  if (p.m <= 16) return launch_split_k<BITS, 1, 1, 4, kSmallWaves>(p, stream);
  if (p.m <= 32) return launch_split_k<BITS, 2, 1, 4, 8>(p, stream);
  return launch_split_k<BITS, KAIO_SK4_RT, 4 / KAIO_SK4_RT, KAIO_SK4_VEC, KAIO_SK4_WAVES>(p, stream);
}

}  // namespace

hipError_t launch_qkv_decode(const QkvProblem& p, hipStream_t stream) {
  static_assert(kDecodeMaxM <= 64, "the widest configuration covers 64 rows");
  static_assert(decode_bn(16) == 64 && decode_bn(32) == 64 && decode_bn(64) == 16 * KAIO_SK4_VEC,
                "strip widths must match the host-side grid computation");
  return p.bits == 8 ? launch_decode_bits<8>(p, stream) : launch_decode_bits<4>(p, stream);
}

}  // namespace kaio
