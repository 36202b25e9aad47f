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
// * Split-K across the waves (wave w takes groups [wG/W, (w+1)G/W)); each
//   wave streams its groups GCHUNK at a time through two register buffers,
//   the next chunk's loads in flight while the current chunk computes.
// * INT4 unpack in nibble-interleaved k order (9 VALU ops per word, once per
//   word whatever RT is); the x fragments are permuted to the same k order in
//   registers.
// * Per group: 4 chained MFMAs per (column set, row tile) into a fresh
//   partial, then acc += partial * scale in f32 (every product exact, as in
//   the tile kernel).
// * The wave partial sums meet in LDS and are added in a fixed order, so
//   results are deterministic; then f32 -> f16 (RNE) and row stores.
// Configurations (rows, columns per strip, waves) are chosen per m so that the
// register file holds two chunks plus the accumulators and the reduction
// buffer stays at 64 KiB: m <= 16: 1 row tile, 64 columns, 16 waves;
// m <= 32: 2, 64, 8; m <= 64: 4, 32, 8.

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
template <> struct WordVec<2> { using T = uint2; };
template <> struct WordVec<4> { using T = uint4; };
template <int V> struct HalfVec { typedef uint16_t T __attribute__((ext_vector_type(V))); };
template <> struct HalfVec<1> { typedef uint16_t T; };

// kFull: n % BN == 0, so every strip is complete and the vector loads of
// weights (VEC words) and scales (VEC halves) stay inside their rows.
// RSPLIT > 1 splits the rows across waves as well: wave w takes row block
// w % RSPLIT (16*RT rows) and reduction part w / RSPLIT of WAVES / RSPLIT.
template <int RT, int RSPLIT, int VEC, int WAVES, bool kFull>
__global__ void __launch_bounds__(WAVES * 64, 1)
qkv_decode_kernel(QkvProblem p, uint32_t nstrips) {
  constexpr int THREADS = WAVES * kWave;
  constexpr int BN = 16 * VEC;                  // columns per strip
  constexpr int KSPLIT = WAVES / RSPLIT;        // waves per row block, splitting the reduction
  constexpr int ROWS = 16 * RT * RSPLIT;        // rows per workgroup
  static_assert(VEC == 1 || VEC == 2 || VEC == 4, "vector width");
  static_assert(KSPLIT * RSPLIT == WAVES, "row split must divide the waves");
  static_assert(KSPLIT * ROWS * BN * 4 <= 65536, "reduction buffer");
  using WV = typename WordVec<VEC>::T;
  __shared__ float red[KSPLIT][ROWS][BN];

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

  const uint32_t* __restrict__ w = q == 0 ? p.w[0] : (q == 1 ? p.w[1] : p.w[2]);
  const uint16_t* __restrict__ s = q == 0 ? p.s[0] : (q == 1 ? p.s[1] : p.s[2]);
  const uint32_t colv = n0 + VEC * l16;     // first of the lane's VEC columns
  // A-operand rows past M repeat row M-1: their outputs are never stored, and
  // MFMA rows do not mix, so no load needs a predicate.
  // (element offsets of the lane's rows: m <= 64 and k < 2^24 keep them below 2^30)
  uint32_t xrow[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const uint32_t row = 16 * RT * rblk + 16 * r + l16;
    xrow[r] = (row < M ? row : M - 1) * K + kb * 8;
  }
  const uint32_t* wlane = w + (size_t)kb * N + colv;   // + (16g + 4ks) * N

  floatx4 acc[VEC][RT];
#pragma unroll
  for (int t = 0; t < VEC; ++t)
#pragma unroll
    for (int r = 0; r < RT; ++r) acc[t][r] = floatx4{0.f, 0.f, 0.f, 0.f};

  struct Chunk {
    uint32_t wv[GCHUNK][4][VEC];
    uint4 xa[GCHUNK][4][RT];
    uint32_t sc[GCHUNK][VEC];
  };
  // Loads of GCHUNK groups starting at g0.  Groups past the wave's range are
  // clamped to its last group (loaded, never used) so that every chunk issues
  // the same loads and the compiler can keep the next chunk in flight.
  auto load_chunk = [&](uint32_t g0, Chunk& c) {
#pragma unroll
    for (int gi = 0; gi < GCHUNK; ++gi) {
      const uint32_t g = (g0 + gi < g_end) ? g0 + gi : g_end - 1;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const size_t roff = ((size_t)g * 16 + ks * 4) * N;
        if (kFull) {
          const WV v = *reinterpret_cast<const WV*>(wlane + roff);
          __builtin_memcpy(c.wv[gi][ks], &v, sizeof(v));
        } else {
#pragma unroll
          for (int t = 0; t < VEC; ++t) c.wv[gi][ks][t] = (colv + t < N) ? wlane[roff + t] : 0u;
        }
#pragma unroll
        for (int r = 0; r < RT; ++r)
          c.xa[gi][ks][r] = *reinterpret_cast<const uint4*>(p.x + xrow[r] + (size_t)g * kGroup + ks * 32);
      }
      if (kFull) {
        using HV = typename HalfVec<VEC>::T;
        const HV sv = *reinterpret_cast<const HV*>(s + (size_t)g * N + colv);
        uint16_t sh[VEC];
        __builtin_memcpy(sh, &sv, sizeof(sv));
#pragma unroll
        for (int t = 0; t < VEC; ++t) c.sc[gi][t] = sh[t];
      } else {
#pragma unroll
        for (int t = 0; t < VEC; ++t) c.sc[gi][t] = (colv + t < N) ? (uint32_t)s[(size_t)g * N + colv + t] : 0u;
      }
    }
  };
  auto compute_chunk = [&](uint32_t g0, const Chunk& c) {
#pragma unroll
    for (int gi = 0; gi < GCHUNK; ++gi) {
      if (g0 + gi < g_end) {   // wave-uniform
        floatx4 part[VEC][RT];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          half8_t a[RT];
#pragma unroll
          for (int r = 0; r < RT; ++r) a[r] = permute_x_like_int4x8(c.xa[gi][ks][r]);
#pragma unroll
          for (int t = 0; t < VEC; ++t) {
            const half8_t b = unpack_int4x8_interleaved(c.wv[gi][ks][t]);
#pragma unroll
            for (int r = 0; r < RT; ++r)
              part[t][r] = mfma16x16x32(a[r], b, ks == 0 ? floatx4{0.f, 0.f, 0.f, 0.f} : part[t][r]);
          }
        }
#pragma unroll
        for (int t = 0; t < VEC; ++t) {
          const float sf = h2f((uint16_t)c.sc[gi][t]);
#pragma unroll
          for (int r = 0; r < RT; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[t][r][i] = __builtin_fmaf(part[t][r][i], sf, acc[t][r][i]);
        }
      }
    }
  };

  if (g_begin < g_end) {
    // two register buffers used ping-pong: chunk c+1 is in flight while
    // chunk c computes.  No chunk past the wave's range is loaded: a load
    // nobody uses would still hold up the wave's final wait.
    Chunk ca, cb;
    load_chunk(g_begin, ca);
    for (uint32_t g0 = g_begin; g0 < g_end; g0 += 2 * GCHUNK) {
      const bool more = g0 + GCHUNK < g_end;   // wave-uniform
      if (more) load_chunk(g0 + GCHUNK, cb);
      compute_chunk(g0, ca);
      if (!more) break;
      if (g0 + 2 * GCHUNK < g_end) load_chunk(g0 + 2 * GCHUNK, ca);
      compute_chunk(g0 + GCHUNK, cb);
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
    if (kFull || gc < N) out[(size_t)row * N + gc] = __builtin_bit_cast(uint16_t, (_Float16)sum);
  }
}

template <int RT, int RSPLIT, int VEC, int WAVES>
hipError_t launch_split_k(const QkvProblem& p, hipStream_t stream) {
  constexpr uint32_t BN = 16 * VEC;
  const uint32_t nstrips = (p.n + BN - 1) / BN;
  const dim3 grid(3 * nstrips), block(WAVES * kWave);
  if (p.n % BN == 0)
    hipLaunchKernelGGL((qkv_decode_kernel<RT, RSPLIT, VEC, WAVES, true>), grid, block, 0, stream, p, nstrips);
  else
    hipLaunchKernelGGL((qkv_decode_kernel<RT, RSPLIT, VEC, WAVES, false>), grid, block, 0, stream, p, nstrips);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qkv_decode(const QkvProblem& p, hipStream_t stream) {
  static_assert(kDecodeMaxM <= 128, "the widest configuration covers 128 rows");
  static_assert(decode_bn(16) == 64 && decode_bn(32) == 64 && decode_bn(64) == 16 * KAIO_SK4_VEC &&
                    decode_bn(128) == 64,
                "strip widths must match the host-side grid computation");
  if (p.m <= 16) return launch_split_k<1, 1, 4, 16>(p, stream);
  if (p.m <= 32) return launch_split_k<2, 1, 4, 8>(p, stream);
  if (p.m <= 64) return launch_split_k<KAIO_SK4_RT, 4 / KAIO_SK4_RT, KAIO_SK4_VEC, KAIO_SK4_WAVES>(p, stream);
  return launch_split_k<KAIO_SK8_RT, 8 / KAIO_SK8_RT, 4, KAIO_SK8_WAVES>(p, stream);
}

}  // namespace kaio
