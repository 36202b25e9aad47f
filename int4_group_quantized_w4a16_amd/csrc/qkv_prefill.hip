// W4A16 fused tri-output QKV projection -- MFMA tile kernel (m > 8).
//
// Operation: kaio-candle 0.2.0, src/qkv_project_int4.rs (module doc and the
// doc comment of qkv_project_int4): one launch computes Q, K and V f16[M,N]
// from a shared f16 x[M,K], three packed-INT4 u32[K/8,N] weights and three
// f16[K/128,N] group scales, accumulating in f32.
//
// gfx950 design
// -------------
// * Workgroup = WAVES waves, tile = 128 rows of x by 16*WAVES columns of EACH
//   output.  Wave w owns columns [16w, 16w+16) of all three outputs and all
//   128 rows, so the waves share one x tile in LDS and never unpack the same
//   weight twice.
// * Everything a group needs -- the x tile, the packed weights, the scales --
//   is staged into an NSTAGE-deep LDS ring with direct global->LDS loads (no
//   registers, no VALU), NSTAGE-1 groups ahead of the MFMAs, one barrier per
//   group.  No register ever waits on a global load, so the only waits on
//   the vector-memory counter are the explicit ones at that barrier.
// * x: chunk kc of row r lands in slot r*16 + (kc ^ (r & 15)), which makes
//   the MFMA A-operand reads bank-conflict free.
// * Weights: one u32 holds the eight consecutive k of one column that a lane
//   feeds to one v_mfma_f32_16x16x32_f16 as its B operand.  Each lane's DMA
//   fetches exactly the word it will multiply into its own LDS slot; the lane
//   reads it back and unpacks it to exact f16 integers in registers.
// * Scales are applied per group in f32: the four MFMAs of a group
//   accumulate a fresh partial sum of x*q (exact small integers times f16
//   activations), then acc += partial * scale.  Rounding q*scale to f16
//   before the MFMA would cost up to 2^-12 relative per product, too much
//   for the f16 output; the partial/scale split keeps every product exact.
// * Epilogue: f32 -> f16 (RNE), transposed through LDS one output at a time,
//   16-byte row stores.

#include "common.hpp"
#include "launch.hpp"

namespace kaio {
namespace {

constexpr int BM = kPrefillBM;          // 128 rows per workgroup
constexpr int RT = BM / 16;             // row tiles per wave
constexpr int KC = kGroup / 8;          // 16-byte chunks per row per group
constexpr int X_CHUNKS = BM * KC;       // 16-byte chunks of x per stage (32 KiB)

#ifndef KAIO_PREFILL_SM
#define KAIO_PREFILL_SM 4
#endif
#ifndef KAIO_PREFILL_SN
#define KAIO_PREFILL_SN 8
#endif

#define KAIO_LDS(p) ((__attribute__((address_space(3))) void*)(p))
#define KAIO_GLOBAL(p) ((__attribute__((address_space(1))) const void*)(p))

// Wait until at most N vector-memory operations of this wave are outstanding,
// then barrier.  Unlike __syncthreads() this does not drain every in-flight
// load (its release fence would wait for the prefetches too); the "memory"
// clobber keeps the compiler from moving LDS accesses across it.  Loads
// return in issue order, so "at most N outstanding" means everything but the
// newest N has landed.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// One stage of the LDS ring, in 16-byte units:
//   x     [X_CHUNKS]                       swizzled rows of x
//   w     [3][4][WAVES][64] u32            word (q, ks) for lane l of wave w
//   s     [3][WAVES][8] u32 pairs of f16   scales of the wave's 16 columns
template <int WAVES>
struct StageLayout {
  static constexpr int kX = 0;
  static constexpr int kW = X_CHUNKS;                          // uint4 offset
  static constexpr int kS = kW + 3 * 4 * WAVES * 64 / 4;
  static constexpr int kSize = kS + (3 * WAVES * 8 + 3) / 4;   // uint4 per stage
};

template <int WAVES, int NSTAGE, bool kAligned>
__global__ void __launch_bounds__(WAVES * 64, 1)
qkv_prefill_kernel(QkvProblem p, uint32_t mtiles) {
  constexpr int THREADS = WAVES * 64;
  constexpr int BN = 16 * WAVES;
  constexpr int XPER = X_CHUNKS / THREADS;       // x loads per thread per stage
  constexpr int OUT_LD = BN + 8;                 // padded f16 row of the epilogue tile
  using L = StageLayout<WAVES>;
  // vector-memory operations per thread per stage: x, 12 weight words, 1 scale pair
  constexpr int VM_PER_STAGE = XPER + 12 + (kAligned ? 1 : 0);
  static_assert(XPER * THREADS == X_CHUNKS, "x stage must split evenly");
  static_assert(BM * OUT_LD * 2 <= NSTAGE * L::kSize * 16, "epilogue tile must fit in the ring");
  static_assert((NSTAGE - 2) * VM_PER_STAGE < 64, "vmcnt range");
  extern __shared__ uint4 smem[];

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t kb = lane >> 4;          // 8-k block of the 32-k MFMA step
  const uint32_t l16 = lane & 15;

  uint32_t tm, tn;
  tile_of<KAIO_PREFILL_SM, KAIO_PREFILL_SN>(blockIdx.x, gridDim.x, mtiles, (p.n + BN - 1) / BN, tm, tn);
  const uint32_t m0 = tm * BM;
  const uint32_t n0 = tn * BN;
  const uint32_t M = p.m, N = p.n, K = p.k;
  const uint32_t G = K / kGroup;

  // ---- per-lane DMA sources ---------------------------------------------------
  const uint16_t* xblk = p.x + (size_t)m0 * K;
  uint32_t xoff[XPER];         // element offset (within row block m0, group 0) of this lane's chunk
#pragma unroll
  for (int i = 0; i < XPER; ++i) {
    const uint32_t slot = (i * WAVES + wave) * 64 + lane;
    const uint32_t row = slot >> 4;
    const uint32_t kc = (slot & 15) ^ (row & 15);
    const uint32_t rowc = (m0 + row < M) ? row : (M - 1 - m0);   // rows past M: any valid row
    xoff[i] = rowc * K + kc * 8;
  }
  const uint32_t col = n0 + wave * 16 + l16;
  const uint32_t colc = col < N ? col : N - 1;   // columns past N are computed, never stored
  const uint32_t woff = kb * N + colc;           // word offset inside a group's 16 packed rows
  // scale pairs: lanes 0..23 fetch the f16 pair (2j, 2j+1) of output q = lane / 8
  const uint32_t sq = lane >> 3, sj = lane & 7;
  const uint32_t scol = n0 + wave * 16 + 2 * sj;
  const uint32_t scolc = (scol < N) ? scol : (N >= 2 ? N - 2 : 0);   // N even on this path
  // select (not index) the scale tensor: a lane-dependent index into the
  // kernel arguments would be fetched from memory
  const uint16_t* s_lane = sq == 0 ? p.s[0] : (sq == 1 ? p.s[1] : p.s[2]);

  auto issue_stage = [&](uint32_t g, int buf) {
    uint4* st = smem + buf * L::kSize;
    const uint16_t* xsrc = xblk + (size_t)g * kGroup;
#pragma unroll
    for (int i = 0; i < XPER; ++i)
      __builtin_amdgcn_global_load_lds(KAIO_GLOBAL(xsrc + xoff[i]),
                                       KAIO_LDS(st + L::kX + (i * WAVES + wave) * 64), 16, 0, 0);
    uint32_t* wst = reinterpret_cast<uint32_t*>(st + L::kW);
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const uint32_t* wg = p.w[q] + (size_t)g * 16 * N;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        __builtin_amdgcn_global_load_lds(KAIO_GLOBAL(wg + ks * 4 * N + woff),
                                         KAIO_LDS(wst + ((q * 4 + ks) * WAVES + wave) * 64), 4, 0, 0);
    }
    if (kAligned) {
      uint32_t* sst = reinterpret_cast<uint32_t*>(st + L::kS);
      if (lane < 24)
        __builtin_amdgcn_global_load_lds(KAIO_GLOBAL(s_lane + (size_t)g * N + scolc),
                                         KAIO_LDS(sst + wave * 24), 4, 0, 0);
    }
  };

  floatx4 acc[RT][3];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int q = 0; q < 3; ++q) acc[r][q] = floatx4{0.f, 0.f, 0.f, 0.f};

  // prologue: stages 0 .. NSTAGE-2 (clamped past the end so every stage issues
  // the same number of loads and the waits below stay exact)
#pragma unroll
  for (int st = 0; st < NSTAGE - 1; ++st) issue_stage((uint32_t)st < G ? st : G - 1, st);

  for (uint32_t g = 0; g < G; ++g) {
    // stage g has landed for this wave; after the barrier, for every wave
    wait_vm_barrier<(NSTAGE - 2) * VM_PER_STAGE>();
    // A clamped stage past the end lands in the slot of group g-1, which
    // nobody reads again.
    issue_stage(g + NSTAGE - 1 < G ? g + NSTAGE - 1 : G - 1, (g + NSTAGE - 1) % NSTAGE);

    const uint4* st = smem + (g % NSTAGE) * L::kSize;
    const uint4* xs = st + L::kX;
    const uint32_t* wst = reinterpret_cast<const uint32_t*>(st + L::kW);
    float sf[3];
    if (kAligned) {
      const uint16_t* sst = reinterpret_cast<const uint16_t*>(st + L::kS);
#pragma unroll
      for (int q = 0; q < 3; ++q) sf[q] = h2f(sst[wave * 48 + q * 16 + l16]);
    } else {
#pragma unroll
      for (int q = 0; q < 3; ++q) sf[q] = h2f(p.s[q][(size_t)g * N + colc]);
    }

    // Software-pipelined tile-major order.  Unpack the group's 12 weight
    // words once; then per row tile r: fetch the A fragments of tile r+1,
    // run tile r's three 4-deep MFMA chains, and fold tile r-1's finished
    // partials into acc while those MFMAs execute.  Scheduling barriers keep
    // the compiler from hoisting every tile's LDS reads (register blow-up).
    half8_t bq[3][4];
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) bq[q][ks] = unpack_int4x8(wst[((q * 4 + ks) * WAVES + wave) * 64 + lane]);
    auto load_a = [&](int r, half8_t (&a)[4]) {
      const uint32_t row = r * 16 + l16;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        a[ks] = __builtin_bit_cast(half8_t, xs[row * KC + ((ks * 4 + kb) ^ (row & 15))]);
    };
    half8_t abuf[2][4];
    floatx4 pbuf[2][3];
    load_a(0, abuf[0]);
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      if (r + 1 < RT) load_a(r + 1, abuf[(r + 1) & 1]);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int q = 0; q < 3; ++q)
          pbuf[r & 1][q] = mfma16x16x32(abuf[r & 1][ks], bq[q][ks],
                                        ks == 0 ? floatx4{0.f, 0.f, 0.f, 0.f} : pbuf[r & 1][q]);
      if (r > 0) {
#pragma unroll
        for (int q = 0; q < 3; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[r - 1][q][i] = __builtin_fmaf(pbuf[(r - 1) & 1][q][i], sf[q], acc[r - 1][q][i]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[RT - 1][q][i] = __builtin_fmaf(pbuf[(RT - 1) & 1][q][i], sf[q], acc[RT - 1][q][i]);
  }

  // ---- epilogue: one output at a time through LDS -----------------------------
  uint16_t* tile = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    __syncthreads();   // ring (or the previous output's tile) no longer read
    // D layout of a 16x16 MFMA tile: lane holds column (lane & 15), rows 4*(lane >> 4) + i
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        tile[(r * 16 + 4 * kb + i) * OUT_LD + wave * 16 + l16] =
            __builtin_bit_cast(uint16_t, (_Float16)acc[r][q][i]);
    __syncthreads();
    uint16_t* out = p.out[q];
    if (kAligned) {
      constexpr int CPR = BN / 8;                    // 16-byte chunks per tile row
#pragma unroll
      for (int i = 0; i < BM * CPR / THREADS; ++i) {
        const uint32_t c = i * THREADS + tid;
        const uint32_t row = c / CPR, cc = c % CPR;
        const uint32_t gr = m0 + row, gc = n0 + cc * 8;
        if (gr < M && gc < N)
          *reinterpret_cast<uint4*>(out + (size_t)gr * N + gc) =
              *reinterpret_cast<const uint4*>(tile + row * OUT_LD + cc * 8);
      }
    } else {
      for (uint32_t e = tid; e < (uint32_t)(BM * BN); e += THREADS) {
        const uint32_t row = e / BN, c = e % BN;
        const uint32_t gr = m0 + row, gc = n0 + c;
        if (gr < M && gc < N) out[(size_t)gr * N + gc] = tile[row * OUT_LD + c];
      }
    }
  }
}

template <int WAVES, int NSTAGE, bool kAligned>
hipError_t launch_variant(const QkvProblem& p, hipStream_t stream) {
  constexpr int BN = 16 * WAVES;
  const uint32_t mtiles = (p.m + BM - 1) / BM;
  const uint32_t ntiles = (p.n + BN - 1) / BN;
  const size_t lds = (size_t)NSTAGE * StageLayout<WAVES>::kSize * 16;
  const dim3 grid(mtiles * ntiles), block(WAVES * 64);
  auto* kern = &qkv_prefill_kernel<WAVES, NSTAGE, kAligned>;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, grid, block, lds, stream, p, mtiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qkv_prefill(const QkvProblem& p, hipStream_t stream) {
  // 16-byte output rows and f16-pair scale loads need n % 8 == 0
  if (p.n % 8 == 0) return launch_variant<kPrefillWaves, kPrefillStages, true>(p, stream);
  return launch_variant<kPrefillWaves, kPrefillStages, false>(p, stream);
}

}  // namespace kaio
