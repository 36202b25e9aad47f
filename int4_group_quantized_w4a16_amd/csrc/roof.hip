// Measurement aid, not an operation of the library: a plain streaming read of
// device memory, the reference an HBM-bound kernel of the same bytes is
// weighed against.
//
// Every thread issues all of its U 16-byte loads before it uses any of them
// (so the whole grid's bytes are in flight at once, as in the decode kernel),
// then XORs them.  The result is stored only if it equals a value the data is
// never built to produce, which keeps the loads live without adding writes.
// Chunk c of workgroup b, load u: index (b * U + u) * THREADS + tid -- each
// wave-wide load covers 1 KiB contiguous.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/kaio_roof.h"

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// NT: the loads carry the non-temporal hint (stream past the caches).
template <int U, int THREADS, bool NT>
__global__ void __launch_bounds__(THREADS) stream_read_kernel(const u32x4_t* __restrict__ src, size_t n16,
                                                              uint32_t* __restrict__ sink) {
  const size_t base = (size_t)blockIdx.x * U * THREADS + threadIdx.x;
  u32x4_t v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const size_t i = base + (size_t)u * THREADS;
    if (i < n16)
      v[u] = NT ? __builtin_nontemporal_load(src + i) : src[i];
    else
      v[u] = u32x4_t{0u, 0u, 0u, 0u};
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  if (acc == 0x9E3779B9u) sink[(size_t)blockIdx.x * THREADS + threadIdx.x] = acc;
}

// One lane reads the shader-clock counter (s_memtime) and the constant-rate
// real-time counter (s_memrealtime) at its start, sleeps in short steps until
// the real-time counter has advanced by `ticks` (or a step limit is reached),
// reads both again and stores the four values.  The ratio of the two deltas,
// times the real-time counter's rate, is the average shader clock of its
// compute unit over that window.  It needs one wave slot and no LDS, so it
// can run beside another kernel's workgroups.
__global__ void __launch_bounds__(64) clock_probe_kernel(unsigned long long* __restrict__ out,
                                                         unsigned long long ticks) {
  if (threadIdx.x != 0) return;
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  unsigned long long r1 = r0, c1 = c0;
  for (uint32_t step = 0; step < (1u << 24) && r1 - r0 < ticks; ++step) {
    __builtin_amdgcn_s_sleep(8);
    r1 = __builtin_amdgcn_s_memrealtime();
    c1 = __builtin_amdgcn_s_memtime();
  }
  out[4 * blockIdx.x + 0] = c1 - c0;
  out[4 * blockIdx.x + 1] = r1 - r0;
  out[4 * blockIdx.x + 2] = r0;
  out[4 * blockIdx.x + 3] = r1;
}

// MFMA work alone at the dense f16 rate: each wave runs 8 independent
// accumulator chains of v_mfma_f32_16x16x32_f16 on register operands (four A
// and four B fragments of hashed values, rotated so that no chain repeats a
// pair within four steps); no memory traffic except one 4-byte store per
// thread at the end.  Its sustained rate is what the matrix cores deliver
// under the chip's power limit when nothing else moves.  The MFMAs are asm
// with the accumulator tied in place (the builtin moves accumulators between
// register files every step); asm is opaque to the compiler's hazard checks,
// so the VALU writes of the operands and the reads of the results are
// separated from the MFMAs by explicit wait states.
__global__ void __launch_bounds__(256) mfma_roof_kernel(float* __restrict__ sink, uint32_t iters) {
  typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
  typedef float floatx4 __attribute__((ext_vector_type(4)));
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  half8_t a[4], b[4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t h = (t * 2654435761u) ^ (uint32_t)(r * 97 + i * 131);
      h ^= h >> 13;
      h *= 0x5bd1e995u;
      h ^= h >> 15;
      a[r][i] = (_Float16)((float)((int)(h & 1023) - 512) * 0.001f);
      b[r][i] = (_Float16)((float)((int)((h >> 10) & 1023) - 512) * 0.001f);
    }
  floatx4 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = floatx4{0.f, 0.f, 0.f, 0.f};
  asm volatile("s_nop 7" ::: "memory");
  for (uint32_t it = 0; it < iters; it += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int c = 0; c < 8; ++c)
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(acc[c]) : "v"(a[(c + u) & 3]), "v"(b[c & 3]));
  }
  asm volatile("s_nop 15\n s_nop 15" ::: "memory");
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) sum += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  sink[t] = sum;
}

// Reads of three packed-weight arrays (`rows` rows x `cols` u32 each, row
// major) by column strips, with non-temporal loads, XORed and stored only on
// a value the data never yields (as above):
//   SC = 64: one workgroup of 16 waves per 64-column strip of one array
//     (3 * cols / 64 workgroups); wave w reads rows [w*rows/16, (w+1)*rows/16),
//     lane (kb, c) the four u32 of columns 4c .. 4c+3 at rows 4i + kb, i.e.
//     256-byte row segments: the weight reads of the decode kernel.
//   SC = 16: one workgroup of 8 waves per 16-column strip of all three
//     arrays (cols / 16 workgroups, neighbouring strips on one XCD); wave w
//     reads rows [w*rows/8, (w+1)*rows/8) of each array, lane (kb, c) the u32
//     of column c: 64-byte row segments.
template <int SC>
__global__ void __launch_bounds__(SC == 64 ? 1024 : 512)
strip_read_kernel(const uint32_t* __restrict__ a0, const uint32_t* __restrict__ a1,
                  const uint32_t* __restrict__ a2, uint32_t rows, uint32_t cols, uint32_t* __restrict__ sink) {
  const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6, kb = lane >> 4, c = lane & 15;
  uint32_t acc = 0;
  if (SC == 64) {
    const uint32_t strips = cols / 64, q = blockIdx.x / strips, s = blockIdx.x % strips;
    const uint32_t* a = q == 0 ? a0 : (q == 1 ? a1 : a2);
    const uint32_t r0 = wave * (rows / 16);
#pragma unroll 8
    for (uint32_t i = 0; i < rows / 64; ++i) {
      const u32x4_t v = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(a + (size_t)(r0 + 4 * i + kb) * cols + 64 * s + 4 * c));
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  } else {
    const uint32_t nb = gridDim.x, per = nb / 8;
    const uint32_t s = blockIdx.x < per * 8 ? (blockIdx.x % 8) * per + blockIdx.x / 8 : blockIdx.x;
    const uint32_t r0 = wave * (rows / 8), col = 16 * s + c;
#pragma unroll 8
    for (uint32_t i = 0; i < rows / 32; ++i) {
      acc ^= __builtin_nontemporal_load(a0 + (size_t)(r0 + 4 * i + kb) * cols + col);
      acc ^= __builtin_nontemporal_load(a1 + (size_t)(r0 + 4 * i + kb) * cols + col);
      acc ^= __builtin_nontemporal_load(a2 + (size_t)(r0 + 4 * i + kb) * cols + col);
    }
  }
  if (acc == 0x9E3779B9u) sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

template <int U, int THREADS>
int launch(const void* src, size_t bytes, void* sink, bool nt, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  const size_t per = (size_t)U * THREADS;
  const size_t blocks = (n16 + per - 1) / per;
  if (blocks == 0 || blocks > (1u << 24)) return 2;
  if (nt)
    hipLaunchKernelGGL((stream_read_kernel<U, THREADS, true>), dim3((uint32_t)blocks), dim3(THREADS), 0, stream,
                       static_cast<const u32x4_t*>(src), n16, static_cast<uint32_t*>(sink));
  else
    hipLaunchKernelGGL((stream_read_kernel<U, THREADS, false>), dim3((uint32_t)blocks), dim3(THREADS), 0, stream,
                       static_cast<const u32x4_t*>(src), n16, static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // namespace

extern "C" {

size_t kaio_roof_sink_bytes(size_t bytes, int loads_per_thread, int threads) {
  if (loads_per_thread < 0) loads_per_thread = -loads_per_thread;
  if (loads_per_thread == 0 || threads <= 0) return 0;
  const size_t per = (size_t)loads_per_thread * threads;
  return ((bytes / 16 + per - 1) / per) * threads * 4;
}

int kaio_roof_stream_read(const void* src, size_t bytes, void* sink, int loads_per_thread, int threads,
                          void* stream) {
  if (!src || !sink || bytes % 16 || (reinterpret_cast<uintptr_t>(src) & 15)) return 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // a negative count selects the same shape with non-temporal loads
  const bool nt = loads_per_thread < 0;
  if (nt) loads_per_thread = -loads_per_thread;
#define KAIO_ROOF_CASE(U, T) \
  if (loads_per_thread == U && threads == T) return launch<U, T>(src, bytes, sink, nt, s);
  KAIO_ROOF_CASE(1, 256) KAIO_ROOF_CASE(2, 256) KAIO_ROOF_CASE(4, 256) KAIO_ROOF_CASE(8, 256)
  KAIO_ROOF_CASE(16, 256) KAIO_ROOF_CASE(4, 512) KAIO_ROOF_CASE(8, 512) KAIO_ROOF_CASE(16, 512)
  KAIO_ROOF_CASE(4, 1024) KAIO_ROOF_CASE(8, 1024) KAIO_ROOF_CASE(16, 1024)
#undef KAIO_ROOF_CASE
  return 2;
}

size_t kaio_roof_strip_sink_bytes(unsigned cols, int strip_cols) {
  if (strip_cols == 64) return (size_t)3 * (cols / 64) * 1024 * 4;
  if (strip_cols == 16) return (size_t)(cols / 16) * 512 * 4;
  return 0;
}

int kaio_roof_strip_read(const void* a0, const void* a1, const void* a2, unsigned rows, unsigned cols,
                         int strip_cols, void* sink, void* stream) {
  if (!a0 || !a1 || !a2 || !sink) return 1;
  if ((reinterpret_cast<uintptr_t>(a0) | reinterpret_cast<uintptr_t>(a1) | reinterpret_cast<uintptr_t>(a2)) & 15)
    return 1;
  if (rows == 0 || cols == 0 || rows % 128 || cols % 64 || rows > (1u << 20) || cols > (1u << 20)) return 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint32_t* p0 = static_cast<const uint32_t*>(a0);
  const uint32_t* p1 = static_cast<const uint32_t*>(a1);
  const uint32_t* p2 = static_cast<const uint32_t*>(a2);
  uint32_t* sk = static_cast<uint32_t*>(sink);
  if (strip_cols == 64)
    hipLaunchKernelGGL(strip_read_kernel<64>, dim3(3 * (cols / 64)), dim3(1024), 0, s, p0, p1, p2, rows, cols, sk);
  else if (strip_cols == 16)
    hipLaunchKernelGGL(strip_read_kernel<16>, dim3(cols / 16), dim3(512), 0, s, p0, p1, p2, rows, cols, sk);
  else
    return 2;
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

int kaio_roof_clock_probe(void* out, unsigned long long ticks, void* stream) {
  if (!out || (reinterpret_cast<uintptr_t>(out) & 7)) return 1;
  hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                     static_cast<unsigned long long*>(out), ticks);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

int kaio_roof_mfma(void* sink, int iters, int workgroups, void* stream) {
  if (!sink || (reinterpret_cast<uintptr_t>(sink) & 3)) return 1;
  if (iters < 4 || iters > (1 << 20) || iters % 4 || workgroups < 1 || workgroups > (1 << 20)) return 1;
  hipLaunchKernelGGL(mfma_roof_kernel, dim3((uint32_t)workgroups), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<float*>(sink), (uint32_t)iters);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

double kaio_roof_mfma_flops(int iters, int workgroups) {
  return (double)workgroups * 4 * iters * 8 * (2.0 * 16 * 16 * 32);
}

int kaio_roof_wall_clock_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
  return khz;
}

}  // extern "C"
