// W4A16 fused tri-output QKV projection -- MFMA tile kernel (m > 64; INT4 from
// m > 32 when the group count divides by 4).
//
// Operation: kaio-candle 0.2.0, src/qkv_project_int4.rs (module doc and the
// doc comment of qkv_project_int4): one launch computes Q, K and V f16[M,N]
// from a shared f16 x[M,K], three packed-INT4 u32[K/8,N] weights and three
// f16[K/128,N] group scales, accumulating in f32.
//
// gfx950 design
// -------------
// * Workgroup = WAVES waves, tile = BM (128, 96 or 64 for small grids) rows
//   of x by 16*WAVES columns of EACH output.  Wave w owns columns
//   [16w, 16w+16) of all three outputs and all BM rows, so the waves share
//   one x tile in LDS and never unpack the same weight twice.  Small grids
//   of 4-wave tiles run two (or four) such sets of waves per workgroup, each
//   over its share of the groups with its own ring, their sums added in LDS
//   at the end; the smallest grids compute one output per workgroup.
// * Everything a group of 128 k needs is staged into LDS rings with direct
//   global->LDS loads (no registers, no VALU): x and the packed weights one
//   group ahead, the scales 32 (or 8) groups at a time.  Each address is a
//   wave-uniform base in SGPRs plus a 32-bit lane offset.  One barrier per
//   group; the only waits on the vector-memory counter are explicit.
// * x: chunk kc of row r lands in slot r*16 + (kc ^ (r & 15)), which makes
//   the MFMA A-operand reads bank-conflict free.  A fragments are read two
//   row tiles ahead of the MFMAs that use them.
// * Weights: one u32 holds the eight consecutive k of one column that a lane
//   feeds to one v_mfma_f32_16x16x32_f16 as its B operand.  Each wave fetches
//   the 16 packed rows x 16 columns it multiplies (one 16-byte load per lane
//   and output when n % 8 == 0), reads its words back and unpacks them to
//   exact f16 values q * 2^-9 in registers (10 VALU ops per word) -- during
//   the last two row tiles of the previous group, so that the unpack
//   overlaps MFMAs; the epilogue takes the factor 2^-9 back, exactly.
// * Scales are applied per group in f32: the four MFMAs of a group
//   accumulate a fresh partial sum of x*q*2^-9 (exact small integers, scaled
//   by a power of two, times f16 activations), then
//   acc += partial * scale (the f16 scale converted inside the FMA;
//   the accumulators hold 2^-9 times the result until the epilogue's
//   exact multiply by 512).  Rounding q*scale to f16
//   before the MFMA would cost up to 2^-12 relative per product, too much
//   for the f16 output; the partial/scale split keeps every product exact.
// * Epilogue: f32 -> f16 (RNE), transposed through LDS one output at a time
//   (unpadded rows, columns swizzled per 4-row group), 16-byte row stores.

#include "common.hpp"
#include "launch.hpp"

namespace kaio {
namespace {

constexpr int KC = kGroup / 8;          // 16-byte chunks per row per group

#ifndef KAIO_PREFILL_XDIST
#define KAIO_PREFILL_XDIST 1
#endif
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

// LDS, in 16-byte units.  x of a group is fetched XDIST groups ahead (ring
// of XDIST+1 slots), the packed weights one group ahead (WSLOTS slots), and
// the scales SCHUNK groups at a time:
//   x  [XDIST+1][X_CHUNKS]            swizzled rows of x
//   w  [WSLOTS][NQ][WAVES][PR][16] u32 packed rows x columns of output q, wave w
//   s  [NQ][WAVES][SCHUNK][16] f16     scales of the wave's 16 columns (n % 8 == 0)
// NQ = outputs per workgroup: 3 (Q, K and V) or 1.
// PR = 16 packed rows per group for INT4, 32 for INT8.  A wave reads only the
// words it loaded itself and has consumed (unpacked into registers) the words
// of group g before the barrier that starts group g, after which it loads
// group g+1: one weight slot is enough, and INT8 (twice the words) uses one so
// that the ring fits in LDS.  INT4 keeps two, or one in a tight ring.
// TIGHT: one weight slot and 8-group scale chunks, for two rings of 128-row
// tiles in one workgroup.
template <int BITS, int WAVES, int XDIST, int BM, int NQ, bool TIGHT = false>
struct RingLayout {
  static constexpr int X_CHUNKS = BM * KC;                // 16-byte chunks of x per stage
  static constexpr int kXSlots = XDIST + 1;
  static constexpr int kWSlots = BITS == 4 && !TIGHT ? 2 : 1;
  static constexpr int kSChunk = TIGHT ? 8 : 32;         // SCHUNK
  static constexpr int kWWords = 256 * (BITS / 4);       // words per output per wave per group
  static constexpr int kWBase = kXSlots * X_CHUNKS;
  static constexpr int kWSize = NQ * WAVES * kWWords / 4;
  static constexpr int kSBase = kWBase + kWSlots * kWSize;
  static constexpr int kSize = kSBase + NQ * WAVES * kSChunk * 16 * 2 / 16;   // uint4
};
constexpr int kLdsBytes = 160 * 1024;   // per workgroup
// the ring of one set of waves: tight when two of the usual ones would not fit
template <int BITS, int WAVES, int XDIST, int BM, int KS, int NQ>
using SetRing = RingLayout<BITS, WAVES, XDIST, BM, NQ,
                           (KS > 1 && KS * RingLayout<BITS, WAVES, XDIST, BM, NQ>::kSize * 16 > kLdsBytes)>;

// LDS row position of packed row r within a wave's [PR][16] word block.  INT8
// B operands take rows 8ks + 2kb + j (k-step ks, 8-k block kb, word j), which
// land on the same banks for kb and kb + 2 unless rows with bit 2 set are
// swapped pairwise (r ^ 1): then the four kb of one read hit four different
// 16-bank windows.  INT4 rows 4ks + kb already do.
template <int BITS>
__device__ __forceinline__ uint32_t wrow_pos(uint32_t r) {
  return BITS == 8 ? r ^ ((r >> 2) & 1u) : r;
}

// A wave-uniform pointer the compiler must treat as opaque (kept in SGPRs):
// stops it from folding the per-lane offsets into 64-bit vector addresses
// hoisted out of the group loop.
__device__ __forceinline__ const char* uniform(const char* p) {
  asm volatile("" : "+s"(p));
  return p;
}

// Direct global -> LDS load of `bytes` (4 or 16) per lane from base + off,
// in the buffer form: while a global (FLAT-encoded) direct load is pending,
// the compiler cannot order the LDS counter and makes every wait for an LDS
// read a full wait, which would drain the fragment prefetch.  The descriptor
// takes the wave-uniform base (SGPRs) with an unlimited range: every offset
// is in bounds by construction.
__device__ __forceinline__ void dma_to_lds(const char* base, uint32_t off, void* lds, int bytes_is_16) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, -1, 0x00020000);
  if (bytes_is_16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, KAIO_LDS(lds), 16, off, 0, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, KAIO_LDS(lds), 4, off, 0, 0, 0);
}

// A fragments of row tile r: lane (kb, l16) reads row 16r + l16, chunk
// 4ks + kb, stored at (4ks + kb) ^ l16 in that row.  xl[ks] points at row
// l16's chunk of k-step ks in the group's x slot, so every tile's reads are
// those four addresses plus an immediate offset.
__device__ __forceinline__ void x_lanes(const uint4* const (&xl)[4], half8_t (&a)[4], int r) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) a[ks] = __builtin_bit_cast(half8_t, xl[ks][r * 16 * KC]);
}
__device__ __forceinline__ void lane_rows(const uint4* __restrict__ xs, uint32_t l16, uint32_t kb,
                                          const uint4* (&xl)[4]) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) xl[ks] = xs + l16 * KC + ((ks * 4 + kb) ^ l16);
}

// acc += p * s with the f16 scale converted inside the FMA (v_fma_mix_f32):
// the accumulators hold 2^-9 times the result (the unpacked weights carry
// that factor), which the epilogue takes back exactly.
template <int NQ>
__device__ __forceinline__ void fold(floatx4 (&acc)[NQ], const floatx4 (&pb)[NQ], const _Float16 (&sf)[NQ]) {
#pragma unroll
  for (int q = 0; q < NQ; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[q][i] = __builtin_fmaf(pb[q][i], (float)sf[q], acc[q][i]);
}

// The MFMA work of one group.
//
// Row tiles 0 .. RT-3 run software-pipelined in tile-major order: fetch the A
// fragments of tile r+2 (three buffers), run tile r's three 4-deep MFMA
// chains into a fresh partial, and fold tile r-1's partials into acc
// (acc += p * s) while those MFMAs execute.  Scheduling barriers keep the
// compiler from hoisting every tile's LDS reads (register blow-up).
//
// The last two tiles run in k-step-major order: once the six MFMAs of step
// ks are issued, the B fragments bq[*][ks] are dead and the next group's
// words are unpacked into them, so the unpack overlaps MFMAs instead of
// stalling the start of the next group.  `next_w` points at this wave's
// next-group words in LDS, `next_s[q]` at its scales; the wait before the
// tail covers them (XPENDING = the x loads issued after them).
template <int BITS, int WAVES, int XPENDING, int RT, int NQ, typename IssueX>
__device__ __forceinline__ void group_mma(floatx4 (&acc)[RT][NQ], half8_t (&bq)[NQ][4], _Float16 (&sf)[NQ],
                                          const uint4* __restrict__ xs, const uint32_t* __restrict__ next_w,
                                          const uint16_t* const (&next_s)[NQ], uint32_t l16, uint32_t kb,
                                          uint32_t lane, IssueX issue_x_part) {
  // A fragments two tiles ahead (three buffers); tiles RT-2 and RT-1 land
  // in buffers (RT-2) % 3 and (RT-1) % 3 during tiles RT-4 and RT-3.
  half8_t abuf[3][4];
  floatx4 pbuf[2][NQ];
  const uint4* xl[4];
  lane_rows(xs, l16, kb, xl);
  x_lanes(xl, abuf[0], 0);
  x_lanes(xl, abuf[1], 1);
#pragma unroll
  for (int r = 0; r < RT - 2; ++r) {
    x_lanes(xl, abuf[(r + 2) % 3], r + 2);
    // a later group's x: load i goes out during tile i mod (RT - 2), so every
    // one of the XPENDING loads is issued before the tail's wait counts them
#pragma unroll
    for (int i = r; i < XPENDING; i += RT - 2) issue_x_part(i);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        pbuf[r & 1][q] = mfma16x16x32(abuf[r % 3][ks], bq[q][ks],
                                      ks == 0 ? floatx4{0.f, 0.f, 0.f, 0.f} : pbuf[r & 1][q]);
    if (r > 0) fold(acc[r - 1], pbuf[(r - 1) & 1], sf);
    __builtin_amdgcn_sched_barrier(0);
  }
  constexpr int T0 = (RT - 2) % 3, T1 = (RT - 1) % 3;
  fold(acc[RT - 3], pbuf[(RT - 3) & 1], sf);
  __builtin_amdgcn_s_setprio(0);
  // this wave's own weights and scales of the next group have landed (only
  // its XPER x loads, issued after them, may still be in flight)
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(XPENDING) : "memory");
  // all of the next group's words and scales are read at once, so that their
  // LDS latency passes under the MFMAs instead of in front of each unpack
  constexpr int WPK = BITS / 4;
  constexpr int WW = 256 * WPK;
  uint32_t nw[NQ][4][WPK];
  uint16_t ns16[NQ];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int j = 0; j < WPK; ++j)
        nw[q][ks][j] = next_w[q * WAVES * WW + wrow_pos<BITS>(WPK * (4 * ks + kb) + j) * 16 + l16];
#pragma unroll
  for (int q = 0; q < NQ; ++q) ns16[q] = *next_s[q];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        pbuf[t][q] = mfma16x16x32(abuf[t == 0 ? T0 : T1][ks], bq[q][ks],
                                  ks == 0 ? floatx4{0.f, 0.f, 0.f, 0.f} : pbuf[t][q]);
#pragma unroll
    for (int q = 0; q < NQ; ++q) bq[q][ks] = unpack_b_scaled<BITS>(nw[q][ks]);
    __builtin_amdgcn_sched_barrier(0);
  }
  fold(acc[RT - 2], pbuf[0], sf);
  fold(acc[RT - 1], pbuf[1], sf);
#pragma unroll
  for (int q = 0; q < NQ; ++q) sf[q] = __builtin_bit_cast(_Float16, ns16[q]);
}

// BITS = 4 (W4A16) or 8 (W8A16: two packed words per 8 k of a column).
// BM = rows of x per workgroup: 128, 96 or 64 (see prefill_form: smaller
// tiles where a grid of larger ones would fill the compute units badly).
// KS = 1, 2 or 4: the workgroup holds KS sets of WAVES waves, each with its
// own ring, that run the same loop over their share of the groups (so KS
// waves share each SIMD and hide each other's waits); the other sets'
// accumulators are added to the first's through LDS before the epilogue, in
// one fixed order.  Needs a group count divisible by KS.
// NQ = 3: each workgroup computes its tile of Q, K and V; NQ = 1: of one of
// them (three times the workgroups, for grids too small to fill the compute
// units otherwise; x is then staged once per output).
template <int BITS, int WAVES, int XDIST, bool kAligned, int BM, int KS, int NQ>
__global__ void __launch_bounds__(KS * WAVES * 64, 1)
qkv_prefill_kernel(QkvProblem p, uint32_t mtiles) {
  constexpr int THREADS = WAVES * 64;            // threads of one set
  constexpr int RT = BM / 16;                    // row tiles per wave
  static_assert(RT >= 3, "two tail tiles after at least one pipelined tile");
  constexpr int WPK = BITS / 4;                  // packed words per 8 k of a column
  constexpr int PR = 16 * WPK;                   // packed rows per group
  constexpr int BN = 16 * WAVES;
  using L = SetRing<BITS, WAVES, XDIST, BM, KS, NQ>;
  constexpr int SCHUNK = L::kSChunk;
  constexpr int X_CHUNKS = L::X_CHUNKS;
  constexpr int XPER = X_CHUNKS / THREADS;       // x loads per thread per stage
  constexpr int OUT_LD = BN;                     // f16 row of the epilogue tile (column-swizzled)
  constexpr int WW = L::kWWords;
  static_assert(XPER * THREADS == X_CHUNKS, "x stage must split evenly");
  static_assert(BM * OUT_LD * 2 <= L::kSize * 16, "epilogue tile must fit in the ring");
  static_assert(BN % 64 == 0, "the epilogue's column swizzle stays inside the tile row");
  static_assert(XPER < 64, "vmcnt range");
  static_assert(KS == 1 || KS == 2 || KS == 4, "one, two or four sets of waves");
  static_assert(KS == 1 || (KS - 1) * WAVES * RT * NQ * 4 * 64 * 4 <= KS * L::kSize * 16,
                "the other sets' sums must fit in LDS");
  static_assert(NQ == 1 || NQ == 3, "one output per workgroup, or all three");
  static_assert(KS * L::kSize * 16 <= kLdsBytes, "rings must fit in LDS");
  extern __shared__ uint4 smem[];

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t wave_id = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t set = wave_id / WAVES;          // which half of the groups (KS = 2)
  const uint32_t wave = wave_id % WAVES;         // wave within its set: its 16 columns
  uint4* const ring = smem + set * L::kSize;
  const uint32_t kb = lane >> 4;          // 8-k block of the 32-k MFMA step
  const uint32_t l16 = lane & 15;

  // NQ = 1: the remapped ids run through the tiles of Q, then K, then V
  const uint32_t ntiles = (p.n + BN - 1) / BN;
  const uint32_t t = xcd_remap(blockIdx.x, gridDim.x);
  const uint32_t q0 = NQ == 1 ? t / (mtiles * ntiles) : 0;   // first output of this workgroup
  uint32_t tm, tn;
  tile_at<KAIO_PREFILL_SM, KAIO_PREFILL_SN>(NQ == 1 ? t % (mtiles * ntiles) : t, mtiles, ntiles, tm, tn);
  const uint32_t m0 = tm * BM;
  const uint32_t n0 = tn * BN;
  const uint32_t M = p.m, N = p.n, K = p.k;
  const uint32_t G = K / kGroup / KS;            // groups of this set
  const uint32_t g0 = set * G;                   // its first group
  const uint32_t* wsrc[NQ];
  const uint16_t* ssrc[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    wsrc[q] = p.w[q0 + q] + (size_t)g0 * PR * N;
    ssrc[q] = p.s[q0 + q] + (size_t)g0 * N;
  }

  // ---- per-lane DMA sources -----------------------------------------------------
  // Each source address is a wave-uniform base plus a 32-bit per-lane byte
  // offset (the host-side size limits keep the offsets below 2^32), which the
  // loads take in their scalar-base form: no per-lane 64-bit address math.
  const char* xblk = reinterpret_cast<const char*>(p.x + (size_t)m0 * K + (size_t)g0 * kGroup);
  uint32_t xoff[XPER];         // byte offset (row block m0, the set's first group) of this lane's chunk
#pragma unroll
  for (int i = 0; i < XPER; ++i) {
    const uint32_t slot = (i * WAVES + wave) * 64 + lane;
    const uint32_t row = slot >> 4;
    const uint32_t kc = (slot & 15) ^ (row & 15);
    const uint32_t rowc = (m0 + row < M) ? row : (M - 1 - m0);   // rows past M: any valid row
    xoff[i] = (rowc * K + kc * 8) * 2;
  }
  const uint32_t col = n0 + wave * 16 + l16;
  const uint32_t colc = col < N ? col : N - 1;   // columns past N are computed, never stored
  // Weights, 16-byte path (n % 8 == 0): load j of lane l fills LDS row
  // position 16j + l/4, columns 4(l % 4) .. +3 of the wave's 16, from the
  // packed row stored there (wrow_pos is its own inverse) -- WPK loads per
  // output per group.  A group of four columns lies wholly inside or wholly
  // past N here.  4-byte path: load i of lane (kb, c) fills row position
  // 4i + kb, column c.
  const uint32_t c4 = n0 + wave * 16 + 4 * (lane & 3);
  const uint32_t woff = kAligned ? (wrow_pos<BITS>(lane >> 2) * N + (c4 < N ? c4 : N - 4)) * 4
                                 : (kb * N + colc) * 4;
  // 4-byte path, INT8: odd loads (row positions with bit 2 set) take rows kb ^ 1
  const uint32_t woff_odd = kAligned ? woff : ((BITS == 8 ? kb ^ 1u : kb) * N + colc) * 4;
  // Scales (n % 8 == 0): lane l fetches the 8 columns 8(l % 2) .. +7 of the
  // wave's 16 for group l / 2 of a chunk -- one 16-byte load per output per
  // SCHUNK groups.
  const uint32_t s8 = n0 + wave * 16 + 8 * (lane & 1);
  const uint32_t s8c = s8 < N ? s8 : N - 8;
  const uint32_t sgi = lane >> 1;     // group within the chunk (lanes 0..2*SCHUNK-1)

  auto xslot = [&](uint32_t g) { return ring + (g % L::kXSlots) * X_CHUNKS; };
  auto wslot = [&](uint32_t g) { return ring + L::kWBase + (g % L::kWSlots) * L::kWSize; };
  auto wave_words = [&](uint32_t g) { return reinterpret_cast<const uint32_t*>(wslot(g)) + wave * WW; };
  uint16_t* const sbuf = reinterpret_cast<uint16_t*>(ring + L::kSBase);

  // Weights of group g (clamped to the last group: a repeat lands in a slot
  // nobody reads) into weight slot g % kWSlots.
  auto issue_w = [&](uint32_t g) {
    const uint32_t gc = g < G ? g : G - 1;
    uint32_t* wst = reinterpret_cast<uint32_t*>(wslot(g)) + wave * WW;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const char* wg = uniform(reinterpret_cast<const char*>(wsrc[q] + (size_t)gc * PR * N));
      if (kAligned) {
#pragma unroll
        for (int j = 0; j < WPK; ++j)
          dma_to_lds(uniform(wg + (size_t)j * 64 * N), woff, wst + q * WAVES * WW + j * 256, 1);
      } else {
#pragma unroll
        for (int i = 0; i < 4 * WPK; ++i)
          dma_to_lds(uniform(wg + (size_t)i * 16 * N), (i & 1) ? woff_odd : woff,
                     wst + q * WAVES * WW + i * 64, 0);
      }
    }
  };
  // Scales of groups c0 .. c0+SCHUNK-1 (clamped to the last group) for the
  // wave's columns into the scale buffer (n % 8 == 0 only).  With shorter
  // chunks only lanes 0 .. 2*SCHUNK-1 load (a lane's bytes land at its own
  // 16-byte offset from the buffer, so the others would overrun it).
  auto issue_s = [&](uint32_t c0) {
    const uint32_t gi = c0 + sgi < G ? sgi : G - 1 - c0;
    const uint32_t off = (gi * N + s8c) * 2;
    if (SCHUNK == 32 || lane < 2 * SCHUNK) {
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        dma_to_lds(uniform(reinterpret_cast<const char*>(ssrc[q] + (size_t)c0 * N)), off,
                   sbuf + (q * WAVES + wave) * SCHUNK * 16, 1);
    }
  };
  // Load i of x of group g (clamped likewise) into x slot g % (XDIST+1).
  auto issue_x_one = [&](uint32_t g, int i) {
    uint4* xst = xslot(g);
    const char* xsrc = uniform(xblk + (size_t)(g < G ? g : G - 1) * kGroup * 2);
    dma_to_lds(xsrc, xoff[i], xst + (i * WAVES + wave) * 64, 1);
  };
  auto issue_x = [&](uint32_t g) {
#pragma unroll
    for (int i = 0; i < XPER; ++i) issue_x_one(g, i);
  };
  // where group g's scales for this lane's column are read from
  auto scale_src = [&](uint32_t g, const uint16_t* (&ns)[NQ]) {
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      ns[q] = kAligned ? sbuf + ((q * WAVES + wave) * SCHUNK + g % SCHUNK) * 16 + l16
                       : ssrc[q] + (size_t)(g < G ? g : G - 1) * N + colc;
  };

  floatx4 acc[RT][NQ];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int q = 0; q < NQ; ++q) acc[r][q] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Prologue: x of groups 0 .. XDIST-1 in flight, group 0 in place and unpacked.
  half8_t bq[NQ][4];
  _Float16 sf[NQ];
  if (kAligned) issue_s(0);
  issue_w(0);
#pragma unroll
  for (int d = 0; d < XDIST; ++d) issue_x(d);
  wait_vm_barrier<0>();
  {
    const uint32_t* w0 = wave_words(0);
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        uint32_t words[WPK];
#pragma unroll
        for (int j = 0; j < WPK; ++j) words[j] = w0[q * WAVES * WW + wrow_pos<BITS>(WPK * (4 * ks + kb) + j) * 16 + l16];
        bq[q][ks] = unpack_b_scaled<BITS>(words);
      }
    const uint16_t* ns[NQ];
    scale_src(0, ns);
#pragma unroll
    for (int q = 0; q < NQ; ++q) sf[q] = __builtin_bit_cast(_Float16, *ns[q]);
  }

  // Per group g, after one barrier: weights of g+1 and x of g+XDIST are
  // issued (weights first), then the tiles of g run, during whose tail the
  // wave unpacks group g+1 (its own loads: it waits with vmcnt(XPER), which
  // leaves only the newest x in flight).  At the barrier x of g is in place
  // everywhere (the per-wave waits since have covered it) and every wave is
  // done with x slot of g-1 and weight slot of g-1, the slots overwritten
  // next.  Every group issues the same loads (clamped past the end), so the
  // counts in the waits are exact; past the last group the tail unpacks a
  // repeat that nothing uses.  (Barrier and loads sit at the top of the
  // body so that no branch follows the MFMA block.)
  for (uint32_t g = 0; g < G; ++g) {
    wait_vm_barrier<(XDIST - 1) * XPER>();
    // Waves w and w+4 share a SIMD and leave each barrier together, so both
    // would reach their VALU-heavy tails at once and leave the MFMA pipe idle.
    // The second of each pair issues first through the pipelined tiles (its
    // priority drops again before its tail), so its tail overlaps the other
    // wave's MFMAs (~3% at 2048 x 4096 x 4096).
    if (KS * WAVES == 8 && wave_id >= 4) __builtin_amdgcn_s_setprio(1);
    issue_w(g + 1);
    // the next scale chunk replaces this one once the tail of g-1 has read
    // the last scale it needed (the scale of g, before the barrier)
    if (kAligned && (g + 1) % SCHUNK == 0 && g + 1 < G) issue_s(g + 1);
    const uint16_t* ns[NQ];
    scale_src(g + 1, ns);
    // x of g + XDIST goes out one load per row tile, between MFMAs
    group_mma<BITS, WAVES, XPER, RT, NQ>(acc, bq, sf, xslot(g), wave_words(g + 1), ns, l16, kb, lane,
                           [&](int i) { issue_x_one(g + XDIST, i); });
  }
  wait_vm_barrier<0>();   // no load is still writing the ring the epilogue reuses

  // ---- the other sets' sums into the first's (KS > 1) -------------------------
  // Wave w of set s holds the same accumulator elements, lane for lane, as
  // wave w of set 0: one f32 per lane and element, lane-contiguous, in the
  // region of set s; set 0 adds them in set order.
  if constexpr (KS > 1) {
    constexpr int E = RT * NQ * 4;
    float* const red = reinterpret_cast<float*>(smem) + wave * E * 64 + lane;
    __syncthreads();   // rings no longer read
    if (set > 0) {
      float* const mine = red + (set - 1) * WAVES * E * 64;
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) mine[((r * NQ + q) * 4 + i) * 64] = acc[r][q][i];
    }
    __syncthreads();
    if (set == 0) {
#pragma unroll
      for (int o = 0; o < KS - 1; ++o)
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
          for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[r][q][i] += red[o * WAVES * E * 64 + ((r * NQ + q) * 4 + i) * 64];
    }
  }

  // ---- epilogue: one output at a time through LDS -----------------------------
  constexpr int TT = KS * THREADS;               // every thread of the workgroup stores
  uint16_t* tile = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    __syncthreads();   // ring (or the sums, or the previous output's tile) no longer read
    // D layout of a 16x16 MFMA tile: lane holds column (lane & 15), rows 4*(lane >> 4) + i.
    // Column c of tile row t sits at c ^ (16 * ((t >> 2) & 3)): the four row
    // groups of one 2-byte store (rows 4 apart) land in four different
    // 32-byte bank windows, and each 16-byte row read stays inside its row.
    if (set == 0) {
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          tile[(r * 16 + 4 * kb + i) * OUT_LD + ((wave * 16 + l16) ^ (16 * kb))] =
              __builtin_bit_cast(uint16_t, (_Float16)(acc[r][q][i] * kUnpackScaledInv));
    }
    __syncthreads();
    uint16_t* out = p.out[q0 + q];
    if (kAligned) {
      constexpr int CPR = BN / 8;                    // 16-byte chunks per tile row
      constexpr int NCH = BM * CPR;                  // 16-byte chunks of the tile
#pragma unroll
      for (int i = 0; i < (NCH + TT - 1) / TT; ++i) {
        const uint32_t c = i * TT + tid;
        const uint32_t row = c / CPR, cc = c % CPR;
        const uint32_t gr = m0 + row, gc = n0 + cc * 8;
        if ((NCH % TT == 0 || c < (uint32_t)NCH) && gr < M && gc < N)
          *reinterpret_cast<uint4*>(out + (size_t)gr * N + gc) =
              *reinterpret_cast<const uint4*>(tile + row * OUT_LD + ((cc * 8) ^ (16 * ((row >> 2) & 3))));
      }
    } else {
      for (uint32_t e = tid; e < (uint32_t)(BM * BN); e += TT) {
        const uint32_t row = e / BN, c = e % BN;
        const uint32_t gr = m0 + row, gc = n0 + c;
        if (gr < M && gc < N) out[(size_t)gr * N + gc] = tile[row * OUT_LD + (c ^ (16 * ((row >> 2) & 3)))];
      }
    }
  }
}

template <int BITS, int WAVES, int XDIST, bool kAligned, int BM, int KS, int NQ>
hipError_t launch_variant(const QkvProblem& p, hipStream_t stream) {
  constexpr int BN = 16 * WAVES;
  const uint32_t mtiles = (p.m + BM - 1) / BM;
  const uint32_t ntiles = (p.n + BN - 1) / BN;
  const size_t lds = (size_t)KS * SetRing<BITS, WAVES, XDIST, BM, KS, NQ>::kSize * 16;
  const dim3 grid(mtiles * ntiles * (NQ == 1 ? 3 : 1)), block(KS * WAVES * 64);
  auto* kern = &qkv_prefill_kernel<BITS, WAVES, XDIST, kAligned, BM, KS, NQ>;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, grid, block, lds, stream, p, mtiles);
  return hipGetLastError();
}

template <int BITS, int WAVES, int BM, int KS, int NQ = 3>
hipError_t launch_aligned_or_not(const QkvProblem& p, hipStream_t stream) {
  // 16-byte output rows and f16-pair scale loads need n % 8 == 0
  return p.n % 8 == 0 ? launch_variant<BITS, WAVES, KAIO_PREFILL_XDIST, true, BM, KS, NQ>(p, stream)
                      : launch_variant<BITS, WAVES, KAIO_PREFILL_XDIST, false, BM, KS, NQ>(p, stream);
}

constexpr uint32_t form_code(PrefillForm f) { return ((f.waves * 1000 + f.bm) * 10 + f.sets) * 10 + f.outs; }

// the form tile_form() picks for this problem
template <int BITS>
hipError_t launch_prefill_bits(const QkvProblem& p, hipStream_t stream) {
  switch (form_code(tile_form(p.m, p.n, p.k, BITS))) {
    case form_code({8, 128, 1, 3}): return launch_aligned_or_not<BITS, 8, 128, 1>(p, stream);
    case form_code({8, 96, 1, 3}): return launch_aligned_or_not<BITS, 8, 96, 1>(p, stream);
    case form_code({4, 128, 2, 3}):
      if constexpr (BITS == 4) return launch_aligned_or_not<BITS, 4, 128, 2>(p, stream);
      break;
    case form_code({4, 96, 2, 3}): return launch_aligned_or_not<BITS, 4, 96, 2>(p, stream);
    case form_code({4, 64, 2, 3}): return launch_aligned_or_not<BITS, 4, 64, 2>(p, stream);
    case form_code({4, 128, 1, 3}): return launch_aligned_or_not<BITS, 4, 128, 1>(p, stream);
    case form_code({4, 96, 1, 3}): return launch_aligned_or_not<BITS, 4, 96, 1>(p, stream);
    case form_code({4, 64, 1, 3}): return launch_aligned_or_not<BITS, 4, 64, 1>(p, stream);
    case form_code({4, 128, 2, 1}): return launch_aligned_or_not<BITS, 4, 128, 2, 1>(p, stream);
    case form_code({4, 96, 2, 1}): return launch_aligned_or_not<BITS, 4, 96, 2, 1>(p, stream);
    case form_code({4, 128, 1, 1}): return launch_aligned_or_not<BITS, 4, 128, 1, 1>(p, stream);
    case form_code({4, 96, 1, 1}): return launch_aligned_or_not<BITS, 4, 96, 1, 1>(p, stream);
    case form_code({4, 64, 4, 1}):
      if constexpr (BITS == 4) return launch_aligned_or_not<BITS, 4, 64, 4, 1>(p, stream);
      break;
    default: break;
  }
  return hipErrorInvalidValue;   // a form without a kernel (tile_form never picks one)
}

}  // namespace

hipError_t launch_qkv_prefill(const QkvProblem& p, hipStream_t stream) {
  return p.bits == 8 ? launch_prefill_bits<8>(p, stream) : launch_prefill_bits<4>(p, stream);
}

}  // namespace kaio
