// W4A16 fused tri-output QKV projection -- memory-bound decode kernel (m <= 8).
//
// Operation: kaio-candle 0.2.0, src/qkv_project_int4.rs (module doc and the
// doc comment of qkv_project_int4); same contract as the tile kernel.
//
// gfx950 design
// -------------
// At m <= 8 the 4-bit weights are almost all of the bytes, and the
// arithmetic intensity (~31 flop/byte) is above the f32 VALU ridge of the
// chip, so the products still run on MFMA: x is the A operand with its rows
// padded to 16 by zeros, the weights the B operand.
// * Workgroup = 8 waves on a 64-column strip of ONE output.  Lane (kb, c)
//   loads one 128-bit vector = the words of columns 4c..4c+3 at packed row
//   kb of a 32-k step: each word is the B operand of one of four MFMAs, whose
//   column c stands for output column 4c + t.  A wave-wide load covers
//   4 packed rows x 256 contiguous bytes.
// * Split-K across the 8 waves (wave w takes groups [wG/8, (w+1)G/8)); every
//   wave issues all its weight, activation and scale loads before its
//   first MFMA, so the whole strip is in flight at once.
// * Per group: 4 chained MFMAs into a fresh partial, then acc += partial *
//   scale in f32 (same exactness argument as the tile kernel).
// * The 8 wave partial sums meet in LDS and are added in a fixed order, so
//   results are deterministic; then f32 -> f16 (RNE) and 128-byte row stores.

#include "common.hpp"
#include "launch.hpp"

namespace kaio {
namespace {

constexpr int WAVES = 8;
constexpr int THREADS = WAVES * kWave;
constexpr int BN = kDecodeBN;          // 64 columns per strip
constexpr int GCHUNK = 4;              // groups loaded per pass of a wave

template <bool kVec>
__global__ void __launch_bounds__(THREADS)
qkv_decode_kernel(QkvProblem p, uint32_t nstrips) {
  __shared__ float red[WAVES][16][BN];

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t wave = tid >> 6;
  const uint32_t kb = lane >> 4;
  const uint32_t l16 = lane & 15;

  const uint32_t q = blockIdx.x / nstrips;
  const uint32_t n0 = (blockIdx.x % nstrips) * BN;
  const uint32_t M = p.m, N = p.n, K = p.k;
  const uint32_t G = K / kGroup;
  const uint32_t g_begin = (uint32_t)(((uint64_t)wave * G) / WAVES);
  const uint32_t g_end = (uint32_t)(((uint64_t)(wave + 1) * G) / WAVES);

  const uint32_t* __restrict__ w = p.w[q];
  const uint16_t* __restrict__ s = p.s[q];
  const uint32_t col4 = n0 + 4 * l16;      // first of the lane's four columns
  const bool row_ok = l16 < M;             // A-operand row of this lane is a real row of x

  floatx4 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (uint32_t g0 = g_begin; g0 < g_end; g0 += GCHUNK) {
    uint4 wv[GCHUNK][4];
    uint4 xa[GCHUNK][4];
    float sc[GCHUNK][4];
#pragma unroll
    for (int gi = 0; gi < GCHUNK; ++gi) {
      const uint32_t g = g0 + gi;
      const bool live = g < g_end;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const size_t r = (size_t)g * 16 + ks * 4 + kb;
        uint4 wq = uint4{0u, 0u, 0u, 0u};
        if (live) {
          if (kVec) {
            if (col4 < N) wq = *reinterpret_cast<const uint4*>(w + r * N + col4);
          } else {
            uint32_t tmp[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) tmp[t] = (col4 + t < N) ? w[r * N + col4 + t] : 0u;
            wq = uint4{tmp[0], tmp[1], tmp[2], tmp[3]};
          }
        }
        wv[gi][ks] = wq;
        uint4 xv = uint4{0u, 0u, 0u, 0u};
        if (live && row_ok)
          xv = *reinterpret_cast<const uint4*>(p.x + (size_t)l16 * K + (size_t)g * kGroup + ks * 32 + kb * 8);
        xa[gi][ks] = xv;
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) sc[gi][t] = 0.f;
      if (live) {
        if (kVec) {
          if (col4 < N) {
            const uint2 sv = *reinterpret_cast<const uint2*>(s + (size_t)g * N + col4);
            sc[gi][0] = h2f((uint16_t)(sv.x & 0xFFFFu));
            sc[gi][1] = h2f((uint16_t)(sv.x >> 16));
            sc[gi][2] = h2f((uint16_t)(sv.y & 0xFFFFu));
            sc[gi][3] = h2f((uint16_t)(sv.y >> 16));
          }
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (col4 + t < N) sc[gi][t] = h2f(s[(size_t)g * N + col4 + t]);
        }
      }
    }
#pragma unroll
    for (int gi = 0; gi < GCHUNK; ++gi) {
      if (g0 + gi < g_end) {
        floatx4 part[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const half8_t a = __builtin_bit_cast(half8_t, xa[gi][ks]);
          const uint32_t words[4] = {wv[gi][ks].x, wv[gi][ks].y, wv[gi][ks].z, wv[gi][ks].w};
#pragma unroll
          for (int t = 0; t < 4; ++t)
            part[t] = mfma16x16x32(a, unpack_int4x8(words[t]),
                                   ks == 0 ? floatx4{0.f, 0.f, 0.f, 0.f} : part[t]);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[t][i] = __builtin_fmaf(part[t][i], sc[gi][t], acc[t][i]);
      }
    }
  }

  // lane holds rows 4*kb + i of MFMA column l16, i.e. output column 4*l16 + t
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][4 * kb + i][4 * l16 + t] = acc[t][i];
  __syncthreads();

  uint16_t* __restrict__ out = p.out[q];
  for (uint32_t e = tid; e < M * BN; e += THREADS) {
    const uint32_t row = e / BN, c = e % BN;
    float sum = 0.f;
#pragma unroll
    for (int wv_ = 0; wv_ < WAVES; ++wv_) sum += red[wv_][row][c];
    const uint32_t gc = n0 + c;
    if (gc < N) out[(size_t)row * N + gc] = __builtin_bit_cast(uint16_t, (_Float16)sum);
  }
}

}  // namespace

hipError_t launch_qkv_decode(const QkvProblem& p, hipStream_t stream) {
  const uint32_t nstrips = (p.n + BN - 1) / BN;
  const dim3 grid(3 * nstrips), block(THREADS);
  if (p.n % 4 == 0)
    hipLaunchKernelGGL(qkv_decode_kernel<true>, grid, block, 0, stream, p, nstrips);
  else
    hipLaunchKernelGGL(qkv_decode_kernel<false>, grid, block, 0, stream, p, nstrips);
  return hipGetLastError();
}

}  // namespace kaio
