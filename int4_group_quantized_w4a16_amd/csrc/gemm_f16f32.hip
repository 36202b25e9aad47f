// Dense f16 x f16 -> f32 matmul, C = A . B.
//
// Operation: kaio-candle 0.2.0, src/matmul_tc_async.rs (module doc;
// MatmulTcAsyncOp::cuda_fwd: A [m,k] and B [k,n] f16, a zeroed [m,n] f32
// output that the kernel writes).  The pages stage tiles global -> shared
// with cp.async on sm_80+; here the tiles go global -> registers -> LDS with
// the next tile's loads in flight during the current tile's MFMAs.
//
// gfx950 design
// -------------
// * Workgroup = 4 waves, tile 256 x 256, k-step 64; each wave owns a
//   128 x 128 sub-tile = 8 x 8 v_mfma_f32_16x16x32_f16 accumulators
//   (256 f32 per lane), which keeps LDS traffic at 16 bytes/clock per SIMD.
// * A [m,k] is K-contiguous, which is the MFMA A-operand order (8
//   consecutive k per lane): stored as is, XOR-swizzled per 16-byte chunk.
// * B [k,n] is N-contiguous; the B operand needs 8 consecutive k of one
//   column.  Each thread loads an 8 (k) x 8 (n) block and transposes it in
//   registers (16-bit shuffles within the thread), so LDS holds B^T [n][k]
//   and the operand reads are plain 16-byte, conflict-free reads.
// * Epilogue: f32 stores straight from the accumulators.

#include "common.hpp"
#include "launch.hpp"

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

// B^T swizzle: chunk kc of column n lives in slot n*8 + (kc ^ bswz(n)).
// Operand reads (8 lanes = 8 consecutive n) and the transposing writes
// (8 lanes = 8 consecutive n-blocks, same j) both hit 8 distinct bank groups.
__device__ __forceinline__ uint32_t bswz(uint32_t n) { return (n ^ (n >> 3)) & 7; }

__device__ __forceinline__ uint32_t lo_pair(uint32_t r0, uint32_t r1) { return (r0 & 0xFFFFu) | (r1 << 16); }
__device__ __forceinline__ uint32_t hi_pair(uint32_t r0, uint32_t r1) { return (r0 >> 16) | (r1 & 0xFFFF0000u); }

// kAligned: k % 8 == 0 and n % 8 == 0, so every 16-byte chunk is either fully
// inside or fully outside the matrix and row starts are 16-byte aligned.
template <bool kAligned>
__device__ __forceinline__ uint4 load_chunk(const uint16_t* base, uint32_t rows, uint32_t cols,
                                            uint32_t r, uint32_t c) {
  if (r >= rows) return uint4{0u, 0u, 0u, 0u};
  if (kAligned) {
    if (c >= cols) return uint4{0u, 0u, 0u, 0u};
    return *reinterpret_cast<const uint4*>(base + (size_t)r * cols + c);
  }
  uint16_t h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = (c + i < cols) ? base[(size_t)r * cols + c + i] : (uint16_t)0;
  return uint4{h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16),
               h[4] | ((uint32_t)h[5] << 16), h[6] | ((uint32_t)h[7] << 16)};
}

template <bool kAligned>
__global__ void __launch_bounds__(THREADS, 1)
gemm_f16f32_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                   float* __restrict__ C, uint32_t M, uint32_t N, uint32_t K, uint32_t mtiles) {
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

  // staging assignment
  // A: chunk c = i*256 + tid -> row c/8, k-chunk c%8
  // B: thread -> 8x8 block: n-block nb = tid % 32, k-block kq = tid / 32
  const uint32_t nb = tid & 31, kq = tid >> 5;

  uint4 ra[8], rb[8];
  auto load_tiles = [&](uint32_t k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t c = i * THREADS + tid;
      const uint32_t row = c >> 3, kc = c & 7;
      const uint32_t gr = m0 + row < M ? m0 + row : M - 1;
      ra[i] = load_chunk<kAligned>(A, M, K, gr, k0 + kc * 8);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      rb[i] = load_chunk<kAligned>(B, K, N, k0 + kq * 8 + i, n0 + nb * 8);
  };
  auto store_tiles = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t c = i * THREADS + tid;
      const uint32_t row = c >> 3, kc = c & 7;
      sm.a[row * KCH + (kc ^ (row & 7))] = ra[i];
    }
    // transpose the 8x8 block: out[j] = column j, 8 consecutive k
    uint32_t d[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) { d[i][0] = rb[i].x; d[i][1] = rb[i].y; d[i][2] = rb[i].z; d[i][3] = rb[i].w; }
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
      const uint32_t n = nb * 8 + j;
      sm.b[n * KCH + (kq ^ bswz(n))] = o;
    }
  };

  floatx4 acc[TT][TT];
#pragma unroll
  for (int r = 0; r < TT; ++r)
#pragma unroll
    for (int c = 0; c < TT; ++c) acc[r][c] = floatx4{0.f, 0.f, 0.f, 0.f};

  const uint32_t nk = (K + BK - 1) / BK;
  if (nk > 0) load_tiles(0);
  for (uint32_t it = 0; it < nk; ++it) {
    __syncthreads();            // previous tile fully consumed
    store_tiles();
    __syncthreads();            // tile visible
    if (it + 1 < nk) load_tiles((it + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      const uint32_t kc = ks * 4 + kb;
      half8_t bf[TT];
#pragma unroll
      for (int c = 0; c < TT; ++c) {
        const uint32_t n = wn * WT + c * 16 + l16;
        bf[c] = __builtin_bit_cast(half8_t, sm.b[n * KCH + (kc ^ bswz(n))]);
      }
#pragma unroll
      for (int r = 0; r < TT; ++r) {
        const uint32_t row = wm * WT + r * 16 + l16;
        const half8_t af = __builtin_bit_cast(half8_t, sm.a[row * KCH + (kc ^ (row & 7))]);
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
        if (gr < M && gc < N) C[(size_t)gr * N + gc] = acc[r][c][i];
      }
    }
}

__global__ void fill_zero_kernel(uint4* __restrict__ dst, size_t n16, uint8_t* __restrict__ tail, uint32_t ntail) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    dst[i] = uint4{0u, 0u, 0u, 0u};
  if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

}  // namespace

hipError_t launch_gemm_f16f32(const uint16_t* a, const uint16_t* b, float* c,
                              uint32_t m, uint32_t n, uint32_t k, hipStream_t stream) {
  const uint32_t mtiles = (m + BM - 1) / BM;
  const uint32_t ntiles = (n + BN - 1) / BN;
  const dim3 grid(mtiles * ntiles), block(THREADS);
  if (k % 8 == 0 && n % 8 == 0)
    hipLaunchKernelGGL(gemm_f16f32_kernel<true>, grid, block, 0, stream, a, b, c, m, n, k, mtiles);
  else
    hipLaunchKernelGGL(gemm_f16f32_kernel<false>, grid, block, 0, stream, a, b, c, m, n, k, mtiles);
  return hipGetLastError();
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
