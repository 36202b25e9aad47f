// Straight-through per-group dequant backward: dq[i, j] = dy[i, j] * scale[i, j / g].
//
// Operation: baracuda-kernels 0.0.1-alpha.68,
// src/quantize/dequantize_per_group_backward.rs (module doc: the formula;
// DequantizePerGroupBackwardArgs: dy and dq [outer, axis], scale
// [outer, axis/g], one dtype; the plan's precision guarantee: deterministic,
// bit-stable).
//
// Each element is ONE correctly rounded multiply in the storage dtype:
// * f32, f64: the IEEE multiply itself (denormals kept, round to nearest even).
// * f16: the product of two f16 values (<= 22 significant bits, magnitude
//   >= 2^-48) is exact in f32; one f32 -> f16 conversion rounds it.
// * bf16: the product of two bf16 values (<= 16 significant bits) is exact in
//   f32 whenever it lies in the f32 normal range; gfx950's f32 -> bf16
//   conversion then rounds it to nearest even.  Below 2^-126 (where f32 itself
//   would round) the product is formed exactly in f64 and rounded to a
//   multiple of 2^-133, the bf16 subnormal spacing.
//
// gfx950 design: HBM-bound streaming.  A workgroup (256 threads) covers
// UNROLL x 256 consecutive 16-byte vectors of one row (UNROLL = 1 measured
// fastest: many small workgroups keep the most loads in flight).  Every
// element is touched once, so the vector stores are non-temporal, and so are
// the vector loads of the 4- and 8-byte types (at [16384, 8192], g = 128:
// f32 175.7 -> 169.9 us, bf16 91.2 -> 86.4 us; non-temporal bf16 loads
// measured slower, 89.7 us).  With
// 16-byte alignment and g a multiple of the
// vector width every vector lies in one group and needs one scale; other
// shapes take an element-wise path with the same arithmetic.

#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace kaio {
namespace {

constexpr int THREADS = 256;
#ifndef KAIO_BWD_UNROLL
#define KAIO_BWD_UNROLL 1
#endif
constexpr int UNROLL = KAIO_BWD_UNROLL;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct F32 {
  using T = float;
  __device__ static T mul(T a, T b) { return a * b; }
};
struct F64 {
  using T = double;
  __device__ static T mul(T a, T b) { return a * b; }
};
struct F16 {
  using T = uint16_t;
  __device__ static T mul(T a, T b) {
    const float p = h2f(a) * h2f(b);                     // exact
    return __builtin_bit_cast(uint16_t, (_Float16)p);   // one RNE rounding
  }
};
struct BF16 {
  using T = uint16_t;
  __device__ static float widen(T a) { return __builtin_bit_cast(float, (uint32_t)a << 16); }
  __device__ static T mul(T a, T b) {
    const float fa = widen(a), fb = widen(b);
    const float p = fa * fb;
    const uint32_t u = __builtin_bit_cast(uint32_t, p);
    if ((u & 0x7F800000u) == 0u && (a & 0x7FFFu) != 0u && (b & 0x7FFFu) != 0u) {
      // f32 subnormal or zero result from non-zero inputs: round the exact
      // f64 product to the bf16 subnormal grid (spacing 2^-133), ties to even.
      const double pd = (double)fa * (double)fb;
      const double k = rint(fabs(pd) * 0x1p133);        // <= 128; 128 is the smallest normal
      return (T)(((u >> 16) & 0x8000u) | (uint32_t)k);
    }
    // the product is exact in f32 here: gfx950's f32 -> bf16 conversion
    // rounds it once, to nearest even (overflow to inf, NaN stays NaN)
    return __builtin_bit_cast(uint16_t, (__bf16)p);
  }
};

template <typename Op, int V, bool kPow2>
__global__ void __launch_bounds__(THREADS)
dequant_bwd_vec_kernel(const typename Op::T* __restrict__ dy, const typename Op::T* __restrict__ sc,
                       typename Op::T* __restrict__ dq, uint32_t axis_v, uint32_t ngroups,
                       uint32_t group, uint32_t gshift, uint32_t blocks_per_row, uint64_t nblocks) {
  using T = typename Op::T;
  struct alignas(16) Vec { T v[V]; };
  for (uint64_t b = blockIdx.x; b < nblocks; b += gridDim.x) {
    const uint64_t row = b / blocks_per_row;
    const uint32_t chunk = (uint32_t)(b - row * blocks_per_row);
    const Vec* src = reinterpret_cast<const Vec*>(dy) + row * axis_v;
    Vec* dst = reinterpret_cast<Vec*>(dq) + row * axis_v;
    const T* srow = sc + row * ngroups;
    Vec in[UNROLL];
    T s[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const uint32_t jv = (chunk * UNROLL + u) * THREADS + threadIdx.x;
      if (jv < axis_v) {
        if (sizeof(T) >= 4)
          in[u] = __builtin_bit_cast(Vec, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + jv));
        else
          in[u] = src[jv];
        const uint32_t j = jv * V;
        s[u] = srow[kPow2 ? (j >> gshift) : (j / group)];
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const uint32_t jv = (chunk * UNROLL + u) * THREADS + threadIdx.x;
      if (jv < axis_v) {
        Vec o;
#pragma unroll
        for (int e = 0; e < V; ++e) o.v[e] = Op::mul(in[u].v[e], s[u]);
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, o), reinterpret_cast<u32x4*>(dst) + jv);
      }
    }
  }
}

template <typename Op>
__global__ void __launch_bounds__(THREADS)
dequant_bwd_scalar_kernel(const typename Op::T* __restrict__ dy, const typename Op::T* __restrict__ sc,
                          typename Op::T* __restrict__ dq, uint64_t total, uint32_t axis,
                          uint32_t ngroups, uint32_t group) {
  const uint64_t stride = (uint64_t)gridDim.x * THREADS;
  for (uint64_t e = (uint64_t)blockIdx.x * THREADS + threadIdx.x; e < total; e += stride) {
    const uint64_t i = e / axis;
    const uint32_t j = (uint32_t)(e - i * axis);
    dq[e] = Op::mul(dy[e], sc[i * ngroups + j / group]);
  }
}

template <typename Op>
hipError_t launch_typed(int64_t outer, int64_t axis, int64_t group, const void* dy_, const void* sc_,
                        void* dq_, hipStream_t stream) {
  using T = typename Op::T;
  constexpr int V = 16 / sizeof(T);
  const T* dy = static_cast<const T*>(dy_);
  const T* sc = static_cast<const T*>(sc_);
  T* dq = static_cast<T*>(dq_);
  const uint32_t ngroups = (uint32_t)(axis / group);
  const bool aligned = ((uintptr_t)dy % 16 == 0) && ((uintptr_t)dq % 16 == 0) && axis % V == 0 &&
                       group % V == 0;
  constexpr uint64_t kMaxGrid = 1u << 20;
  if (aligned) {
    const uint32_t axis_v = (uint32_t)(axis / V);
    const uint32_t per_block = THREADS * UNROLL;
    const uint32_t bpr = (axis_v + per_block - 1) / per_block;
    const uint64_t nblocks = (uint64_t)outer * bpr;
    const uint32_t grid = (uint32_t)(nblocks < kMaxGrid ? nblocks : kMaxGrid);
    const bool pow2 = (group & (group - 1)) == 0;
    const uint32_t gshift = pow2 ? (uint32_t)__builtin_ctzll((unsigned long long)group) : 0u;
    if (pow2)
      hipLaunchKernelGGL((dequant_bwd_vec_kernel<Op, V, true>), dim3(grid), dim3(THREADS), 0, stream,
                         dy, sc, dq, axis_v, ngroups, (uint32_t)group, gshift, bpr, nblocks);
    else
      hipLaunchKernelGGL((dequant_bwd_vec_kernel<Op, V, false>), dim3(grid), dim3(THREADS), 0, stream,
                         dy, sc, dq, axis_v, ngroups, (uint32_t)group, gshift, bpr, nblocks);
  } else {
    const uint64_t total = (uint64_t)outer * (uint64_t)axis;
    uint64_t blocks = (total + THREADS - 1) / THREADS;
    if (blocks > kMaxGrid) blocks = kMaxGrid;
    hipLaunchKernelGGL((dequant_bwd_scalar_kernel<Op>), dim3((uint32_t)blocks), dim3(THREADS), 0, stream,
                       dy, sc, dq, total, (uint32_t)axis, ngroups, (uint32_t)group);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dequant_group_bwd(kaio_dtype dtype, int64_t outer, int64_t axis, int64_t group,
                                    const void* dy, const void* scale, void* dq, hipStream_t stream) {
  switch (dtype) {
    case KAIO_DTYPE_F32: return launch_typed<F32>(outer, axis, group, dy, scale, dq, stream);
    case KAIO_DTYPE_F64: return launch_typed<F64>(outer, axis, group, dy, scale, dq, stream);
    case KAIO_DTYPE_F16: return launch_typed<F16>(outer, axis, group, dy, scale, dq, stream);
    case KAIO_DTYPE_BF16: return launch_typed<BF16>(outer, axis, group, dy, scale, dq, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace kaio
