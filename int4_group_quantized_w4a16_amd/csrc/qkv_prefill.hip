// W4A16 fused tri-output QKV projection -- MFMA tile kernel (m > 8).
//
// Operation: kaio-candle 0.2.0, src/qkv_project_int4.rs (module doc and the
// doc comment of qkv_project_int4): one launch computes Q, K and V f16[M,N]
// from a shared f16 x[M,K], three packed-INT4 u32[K/8,N] weights and three
// f16[K/128,N] group scales, accumulating in f32.
//
// gfx950 design
// -------------
// * Workgroup = 4 waves, tile = 128 rows of x by 64 columns of EACH output.
//   Wave w owns columns [16w, 16w+16) of all three outputs and all 128 rows,
//   so the four waves share one x tile in LDS and never unpack the same
//   weight twice.
// * x is staged per quantization group (128 k) into a double-buffered,
//   XOR-swizzled LDS tile (16-byte chunk kc of row r lives in slot
//   r*16 + (kc ^ (r & 15)), so the MFMA A reads are bank-conflict free).
// * Weights go straight from global memory to registers: one u32 holds the
//   eight consecutive k of one column that a lane feeds to one
//   v_mfma_f32_16x16x32_f16 as its B operand, so each lane loads exactly the
//   words it multiplies and unpacks them to exact f16 integers in registers.
// * Scales are applied per group in f32: the four MFMAs of a group
//   accumulate a fresh partial sum of x*q (exact small integers times f16
//   activations), then acc += partial * scale.  Rounding q*scale to f16
//   before the MFMA would cost up to 2^-12 relative per product, too much
//   for the f16 output; the partial/scale split keeps every product exact.
// * Epilogue: f32 -> f16 (RNE), transposed through LDS, 16-byte row stores.

#include "common.hpp"
#include "launch.hpp"

namespace kaio {
namespace {

constexpr int BM = kPrefillBM;          // 128
constexpr int BN = kPrefillBN;          // 64
constexpr int THREADS = 256;
constexpr int RT = BM / 16;             // row tiles per wave
constexpr int KC = kGroup / 8;          // 16-byte chunks per row per group
constexpr int XPER = BM * KC / THREADS; // chunks staged per thread per group
constexpr int OUT_LD = BN + 8;          // padded row of the epilogue tile (f16)

static_assert(XPER * THREADS == BM * KC, "x tile must split evenly");

struct alignas(16) SmemPrefill {
  union {
    uint4 x[2][BM * KC];
    uint16_t out[3][BM][OUT_LD];
  };
};

template <bool kVecOut>
__global__ void __launch_bounds__(THREADS, 1)
qkv_prefill_kernel(QkvProblem p, uint32_t mtiles) {
  __shared__ SmemPrefill sm;

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t wave = tid >> 6;
  const uint32_t kb = lane >> 4;          // 8-k block of the 32-k MFMA step
  const uint32_t l16 = lane & 15;

  const uint32_t b = xcd_remap(blockIdx.x, gridDim.x);
  const uint32_t m0 = (b % mtiles) * BM;
  const uint32_t n0 = (b / mtiles) * BN;
  const uint32_t M = p.m, N = p.n, K = p.k;
  const uint32_t G = K / kGroup;

  const uint32_t col = n0 + wave * 16 + l16;
  const size_t colc = col < N ? col : N - 1;   // clamp: columns past N are computed, never stored

  floatx4 acc[RT][3];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int q = 0; q < 3; ++q) acc[r][q] = floatx4{0.f, 0.f, 0.f, 0.f};

  if (G > 0) {
    uint4 xr[XPER];
    uint32_t wr[3][4], wn[3][4];
    float sr[3], sn[3];

    auto load_x = [&](uint32_t g) {
#pragma unroll
      for (int i = 0; i < XPER; ++i) {
        const uint32_t c = i * THREADS + tid;
        const uint32_t row = c >> 4, kc = c & 15;
        const uint32_t grow = (m0 + row < M) ? m0 + row : M - 1;
        xr[i] = *reinterpret_cast<const uint4*>(p.x + (size_t)grow * K + (size_t)g * kGroup + kc * 8);
      }
    };
    auto store_x = [&](int buf) {
#pragma unroll
      for (int i = 0; i < XPER; ++i) {
        const uint32_t c = i * THREADS + tid;
        const uint32_t row = c >> 4, kc = c & 15;
        sm.x[buf][row * KC + (kc ^ (row & 15))] = xr[i];
      }
    };
    auto load_w = [&](uint32_t g, uint32_t (&w)[3][4], float (&s)[3]) {
#pragma unroll
      for (int q = 0; q < 3; ++q) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const size_t r = (size_t)g * 16 + ks * 4 + kb;
          w[q][ks] = p.w[q][r * N + colc];
        }
        s[q] = h2f(p.s[q][(size_t)g * N + colc]);
      }
    };

    load_x(0);
    load_w(0, wr, sr);
    store_x(0);

    for (uint32_t g = 0; g < G; ++g) {
      __syncthreads();
      const int buf = g & 1;
      const bool more = g + 1 < G;
      if (more) {
        load_x(g + 1);
        load_w(g + 1, wn, sn);
      }
      const uint4* xs = sm.x[buf];
      floatx4 part[RT][3];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        half8_t bq[3];
#pragma unroll
        for (int q = 0; q < 3; ++q) bq[q] = unpack_int4x8(wr[q][ks]);
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          const uint32_t row = r * 16 + l16;
          const uint32_t kc = ks * 4 + kb;
          const half8_t a = __builtin_bit_cast(half8_t, xs[row * KC + (kc ^ (row & 15))]);
#pragma unroll
          for (int q = 0; q < 3; ++q) {
            part[r][q] = mfma16x16x32(a, bq[q], ks == 0 ? floatx4{0.f, 0.f, 0.f, 0.f} : part[r][q]);
          }
        }
      }
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int q = 0; q < 3; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[r][q][i] = __builtin_fmaf(part[r][q][i], sr[q], acc[r][q][i]);
      if (more) {
        store_x(buf ^ 1);
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          sr[q] = sn[q];
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) wr[q][ks] = wn[q][ks];
        }
      }
    }
  }

  __syncthreads();   // every wave is done with the x buffers
  // D layout of a 16x16 MFMA tile: lane holds column (lane & 15), rows 4*(lane >> 4) + i.
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t row = r * 16 + 4 * kb + i;
        sm.out[q][row][wave * 16 + l16] = __builtin_bit_cast(uint16_t, (_Float16)acc[r][q][i]);
      }
  __syncthreads();

  if (kVecOut) {
    constexpr int CH = BM * BN / 8;   // 16-byte chunks per output tile
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
      for (int i = 0; i < CH / THREADS; ++i) {
        const uint32_t c = i * THREADS + tid;
        const uint32_t row = c >> 3, cc = c & 7;
        const uint32_t gr = m0 + row, gc = n0 + cc * 8;
        if (gr < M && gc < N)
          *reinterpret_cast<uint4*>(p.out[q] + (size_t)gr * N + gc) =
              *reinterpret_cast<const uint4*>(&sm.out[q][row][cc * 8]);
      }
  } else {
    for (int q = 0; q < 3; ++q)
      for (uint32_t e = tid; e < (uint32_t)(BM * BN); e += THREADS) {
        const uint32_t row = e / BN, c = e % BN;
        const uint32_t gr = m0 + row, gc = n0 + c;
        if (gr < M && gc < N) p.out[q][(size_t)gr * N + gc] = sm.out[q][row][c];
      }
  }
}

}  // namespace

hipError_t launch_qkv_prefill(const QkvProblem& p, hipStream_t stream) {
  const uint32_t mtiles = (p.m + BM - 1) / BM;
  const uint32_t ntiles = (p.n + BN - 1) / BN;
  const dim3 grid(mtiles * ntiles), block(THREADS);
  if (p.n % 8 == 0)
    hipLaunchKernelGGL(qkv_prefill_kernel<true>, grid, block, 0, stream, p, mtiles);
  else
    hipLaunchKernelGGL(qkv_prefill_kernel<false>, grid, block, 0, stream, p, mtiles);
  return hipGetLastError();
}

}  // namespace kaio
