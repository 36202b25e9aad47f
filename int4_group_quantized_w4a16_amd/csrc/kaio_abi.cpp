// C ABI entry points: host-side validation, device check, dispatch.
// Every check here runs before any HIP call, so argument errors are reported
// the same way with or without a GPU.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "launch.hpp"

static_assert(kaio::kGemmBwdScratchBytes == KAIO_GEMM_BWD_NOALLOC_MAX_BYTES,
              "the header's limit must match the static buffer");

namespace {

thread_local std::string g_last_error;

kaio_status fail(kaio_status st, const char* op, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = std::string("kaio::") + op + ": " + buf;
  return st;
}

kaio_status ok() {
  g_last_error.clear();
  return KAIO_OK;
}

// a*b*c as bytes, false when it does not fit comfortably in the address space
bool bytes_of(uint64_t a, uint64_t b, uint64_t c, uint64_t* out) {
  unsigned __int128 v = (unsigned __int128)a * b * c;
  if (v >= ((unsigned __int128)1 << 62)) return false;
  *out = (uint64_t)v;
  return true;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
  const char* name;
};

// first pair (output, other) whose byte ranges intersect; empty ranges never do
const Range* overlap(const Range* outs, int nouts, const Range* ins, int nins, const Range** other) {
  for (int i = 0; i < nouts; ++i) {
    if (outs[i].lo == outs[i].hi) continue;
    for (int j = 0; j < nins; ++j) {
      if (ins[j].lo == ins[j].hi) continue;
      if (outs[i].lo < ins[j].hi && ins[j].lo < outs[i].hi) { *other = &ins[j]; return &outs[i]; }
    }
    for (int j = i + 1; j < nouts; ++j) {
      if (outs[j].lo == outs[j].hi) continue;
      if (outs[i].lo < outs[j].hi && outs[j].lo < outs[i].hi) { *other = &outs[j]; return &outs[i]; }
    }
  }
  return nullptr;
}

Range range(const void* p, uint64_t bytes, const char* name) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + (uintptr_t)bytes, name};
}

// Device check, cached per device ordinal: the current device must be gfx950.
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_state[kMaxDevices];  // 0 unknown, 1 ok, 2 bad

kaio_status check_device(const char* op) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0)
    return fail(KAIO_ERR_DEVICE, op, "no HIP device available (%s); there is no CPU fallback",
                hipGetErrorString(e));
  if (dev >= kMaxDevices) return fail(KAIO_ERR_DEVICE, op, "device ordinal %d out of range", dev);
  int st = g_device_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(KAIO_ERR_DEVICE, op, "hipGetDeviceProperties failed: %s", hipGetErrorString(e));
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_device_state[dev].store(st, std::memory_order_release);
  }
  if (st != 1) {
    hipDeviceProp_t prop;
    const char* arch = (hipGetDeviceProperties(&prop, dev) == hipSuccess) ? prop.gcnArchName : "?";
    return fail(KAIO_ERR_DEVICE, op, "device %d is %s; this library is built for gfx950 (MI355X) only",
                dev, arch);
  }
  return KAIO_OK;
}

kaio_status launched(const char* op, hipError_t e) {
  if (e != hipSuccess) return fail(KAIO_ERR_LAUNCH, op, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

// kaio_gemm_f16f32_bwd and its allocation-free variant (noalloc: f16(grad) goes
// to the library's static per-device buffer instead of the caller's workspace).
kaio_status gemm_bwd(const char* op, const void* a, const void* b, const float* grad, void* grad_a,
                     void* grad_b, uint32_t m, uint32_t n, uint32_t k, bool noalloc, void* workspace,
                     size_t workspace_bytes, void* stream) {
  uint64_t a_bytes = 0, b_bytes = 0, g_bytes = 0, g16_bytes = 0;
  const uint64_t wgs_a = (uint64_t)((m + kaio::kGemmBM - 1) / kaio::kGemmBM) *
                         ((k + kaio::kGemmBN - 1) / kaio::kGemmBN);
  const uint64_t wgs_b = (uint64_t)((k + kaio::kGemmBM - 1) / kaio::kGemmBM) *
                         ((n + kaio::kGemmBN - 1) / kaio::kGemmBN);
  if (!bytes_of(m, k, 2, &a_bytes) || !bytes_of(k, n, 2, &b_bytes) || !bytes_of(m, n, 4, &g_bytes) ||
      !bytes_of(m, n, 2, &g16_bytes) || wgs_a > kaio::kMaxWorkgroups || wgs_b > kaio::kMaxWorkgroups)
    return fail(KAIO_ERR_INVALID_PROBLEM, op, "problem too large for one launch (m=%u, n=%u, k=%u)", m, n, k);
  if (noalloc && g16_bytes > kaio::kGemmBwdScratchBytes)
    return fail(KAIO_ERR_UNSUPPORTED, op,
                "f16(grad) needs m*n*2 = %llu bytes, more than the static buffer of %llu bytes "
                "(use kaio_gemm_f16f32_bwd with a workspace)",
                (unsigned long long)g16_bytes, (unsigned long long)kaio::kGemmBwdScratchBytes);
  if (k == 0) return ok();
  if (m > 0 && !grad_a) return fail(KAIO_ERR_INVALID_ARGUMENT, op, "output grad_a is null");
  if (n > 0 && !grad_b) return fail(KAIO_ERR_INVALID_ARGUMENT, op, "output grad_b is null");
  const bool empty = m == 0 || n == 0;   // both gradients are the empty sum
  if (!empty) {
    if (!a) return fail(KAIO_ERR_INVALID_ARGUMENT, op, "input a is null");
    if (!b) return fail(KAIO_ERR_INVALID_ARGUMENT, op, "input b is null");
    if (!grad) return fail(KAIO_ERR_INVALID_ARGUMENT, op, "input grad is null");
    if (!noalloc && !workspace) return fail(KAIO_ERR_INVALID_ARGUMENT, op, "workspace is null");
    if (!noalloc && workspace_bytes < g16_bytes)
      return fail(KAIO_ERR_INVALID_ARGUMENT, op, "workspace_bytes (%zu) < %llu needed", workspace_bytes,
                  (unsigned long long)g16_bytes);
  }
  if (m > 0 && !aligned16(grad_a)) return fail(KAIO_ERR_INVALID_ARGUMENT, op, "output grad_a is not 16-byte aligned");
  if (n > 0 && !aligned16(grad_b)) return fail(KAIO_ERR_INVALID_ARGUMENT, op, "output grad_b is not 16-byte aligned");
  if (!empty) {
    if (!aligned16(a)) return fail(KAIO_ERR_INVALID_ARGUMENT, op, "input a is not 16-byte aligned");
    if (!aligned16(b)) return fail(KAIO_ERR_INVALID_ARGUMENT, op, "input b is not 16-byte aligned");
    if (!aligned16(grad)) return fail(KAIO_ERR_INVALID_ARGUMENT, op, "input grad is not 16-byte aligned");
    if (!noalloc && !aligned16(workspace)) return fail(KAIO_ERR_INVALID_ARGUMENT, op, "workspace is not 16-byte aligned");
  }
  // written: grad_a, grad_b, and (when not empty) the workspace
  const Range ro[3] = {range(grad_a, a_bytes, "grad_a"), range(grad_b, b_bytes, "grad_b"),
                       range(empty || noalloc ? nullptr : workspace, empty || noalloc ? 0 : g16_bytes,
                             "workspace")};
  const Range ri[3] = {range(empty ? nullptr : a, empty ? 0 : a_bytes, "a"),
                       range(empty ? nullptr : b, empty ? 0 : b_bytes, "b"),
                       range(empty ? nullptr : grad, empty ? 0 : g_bytes, "grad")};
  const Range* other = nullptr;
  if (const Range* o = overlap(ro, 3, ri, 3, &other))
    return fail(KAIO_ERR_INVALID_ARGUMENT, op, "%s overlaps %s", o->name, other->name);
  if (kaio_status st = check_device(op)) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (empty) {
    if (m > 0)
      if (hipError_t e = kaio::launch_fill_zero(grad_a, a_bytes, s)) return launched(op, e);
    if (n > 0)
      if (hipError_t e = kaio::launch_fill_zero(grad_b, b_bytes, s)) return launched(op, e);
    return launched(op, hipSuccess);
  }
  if (noalloc)
    return launched(op, kaio::launch_gemm_f16f32_bwd_noalloc(
                            static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(b), grad,
                            static_cast<uint16_t*>(grad_a), static_cast<uint16_t*>(grad_b), m, n, k, s));
  return launched(op, kaio::launch_gemm_f16f32_bwd(
                          static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(b), grad,
                          static_cast<uint16_t*>(grad_a), static_cast<uint16_t*>(grad_b),
                          static_cast<uint16_t*>(workspace), m, n, k, s));
}

// kaio_qkv_w4a16 (bits 4: u32[k/8, n] weights) and kaio_qkv_w8a16 (bits 8:
// u32[k/4, n] weights): the same validation, the same kernels templated on
// the weight width.
kaio_status qkv(const char* op, uint32_t bits, const void* x, const uint32_t* w_q, const uint32_t* w_k,
                const uint32_t* w_v, const void* s_q, const void* s_k, const void* s_v, void* q, void* k_out,
                void* v, uint32_t m, uint32_t n, uint32_t k, uint32_t group_size, void* stream) {
  if (group_size != 128)
    return fail(KAIO_ERR_UNSUPPORTED, op, "group_size (%u) must be 128 (locked by the kernel contract)",
                group_size);
  if (k % 128 != 0)
    return fail(KAIO_ERR_INVALID_PROBLEM, op, "K (%u) must be a multiple of group_size (128)", k);
  if (m == 0 || n == 0) return ok();

  uint64_t out_bytes = 0, x_bytes = 0, w_bytes = 0, s_bytes = 0;
  const bool decode = kaio::qkv_split_k(m, k, bits);
  const uint64_t wgs = decode ? 3ull * ((n + kaio::decode_bn(m) - 1) / kaio::decode_bn(m))
                              : kaio::prefill_wgs(kaio::tile_form(m, n, k, bits), m, n);
  if (!bytes_of(m, n, 2, &out_bytes) || !bytes_of(m, k, 2, &x_bytes) || !bytes_of(k / (32 / bits), n, 4, &w_bytes) ||
      !bytes_of(k / 128, n, 2, &s_bytes) || wgs > kaio::kMaxWorkgroups || n >= kaio::kMaxN ||
      k >= kaio::kMaxK)
    return fail(KAIO_ERR_INVALID_PROBLEM, op, "problem too large for one launch (m=%u, n=%u, k=%u)", m, n, k);

  const void* ins[7] = {x, w_q, w_k, w_v, s_q, s_k, s_v};
  static const char* in_names[7] = {"x", "w_q_packed", "w_k_packed", "w_v_packed",
                                    "scales_q", "scales_k", "scales_v"};
  void* outs[3] = {q, k_out, v};
  static const char* out_names[3] = {"q", "k", "v"};
  for (int i = 0; i < 3; ++i)
    if (!outs[i]) return fail(KAIO_ERR_INVALID_ARGUMENT, op, "output %s is null", out_names[i]);
  if (k > 0)
    for (int i = 0; i < 7; ++i)
      if (!ins[i]) return fail(KAIO_ERR_INVALID_ARGUMENT, op, "input %s is null", in_names[i]);
  for (int i = 0; i < 3; ++i)
    if (!aligned16(outs[i]))
      return fail(KAIO_ERR_INVALID_ARGUMENT, op, "output %s is not 16-byte aligned", out_names[i]);
  if (k > 0)
    for (int i = 0; i < 7; ++i)
      if (!aligned16(ins[i]))
        return fail(KAIO_ERR_INVALID_ARGUMENT, op, "input %s is not 16-byte aligned", in_names[i]);

  const Range ro[3] = {range(q, out_bytes, "q"), range(k_out, out_bytes, "k"), range(v, out_bytes, "v")};
  const Range ri[7] = {range(x, x_bytes, "x"),           range(w_q, w_bytes, "w_q_packed"),
                       range(w_k, w_bytes, "w_k_packed"), range(w_v, w_bytes, "w_v_packed"),
                       range(s_q, s_bytes, "scales_q"),   range(s_k, s_bytes, "scales_k"),
                       range(s_v, s_bytes, "scales_v")};
  const Range* other = nullptr;
  if (const Range* o = overlap(ro, 3, ri, 7, &other))
    return fail(KAIO_ERR_INVALID_ARGUMENT, op, "output %s overlaps %s", o->name, other->name);

  if (kaio_status st = check_device(op)) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // start from a clean error state
  if (k == 0) {
    for (int i = 0; i < 3; ++i)
      if (hipError_t e = kaio::launch_fill_zero(outs[i], out_bytes, s)) return launched(op, e);
    return ok();
  }
  kaio::QkvProblem p;
  p.x = static_cast<const uint16_t*>(x);
  p.w[0] = w_q; p.w[1] = w_k; p.w[2] = w_v;
  p.s[0] = static_cast<const uint16_t*>(s_q);
  p.s[1] = static_cast<const uint16_t*>(s_k);
  p.s[2] = static_cast<const uint16_t*>(s_v);
  p.out[0] = static_cast<uint16_t*>(q);
  p.out[1] = static_cast<uint16_t*>(k_out);
  p.out[2] = static_cast<uint16_t*>(v);
  p.m = m; p.n = n; p.k = k;
  p.bits = bits;
  return launched(op, decode ? kaio::launch_qkv_decode(p, s) : kaio::launch_qkv_prefill(p, s));
}

}  // namespace

extern "C" {

kaio_status kaio_qkv_w4a16(const void* x, const uint32_t* w_q, const uint32_t* w_k, const uint32_t* w_v,
                           const void* s_q, const void* s_k, const void* s_v, void* q, void* k_out,
                           void* v, uint32_t m, uint32_t n, uint32_t k, uint32_t group_size,
                           void* stream) {
  return qkv("qkv_w4a16", 4, x, w_q, w_k, w_v, s_q, s_k, s_v, q, k_out, v, m, n, k, group_size, stream);
}

kaio_status kaio_qkv_w8a16(const void* x, const uint32_t* w_q, const uint32_t* w_k, const uint32_t* w_v,
                           const void* s_q, const void* s_k, const void* s_v, void* q, void* k_out,
                           void* v, uint32_t m, uint32_t n, uint32_t k, uint32_t group_size,
                           void* stream) {
  return qkv("qkv_w8a16", 8, x, w_q, w_k, w_v, s_q, s_k, s_v, q, k_out, v, m, n, k, group_size, stream);
}

kaio_status kaio_gemm_f16f32(const void* a, const void* b, float* c, uint32_t m, uint32_t n, uint32_t k,
                             void* stream) {
  static const char* op = "gemm_f16f32";
  if (m == 0 || n == 0) return ok();
  uint64_t c_bytes = 0, a_bytes = 0, b_bytes = 0;
  const uint64_t wgs = (uint64_t)((m + kaio::kGemmBM - 1) / kaio::kGemmBM) *
                       ((n + kaio::kGemmBN - 1) / kaio::kGemmBN);
  if (!bytes_of(m, n, 4, &c_bytes) || !bytes_of(m, k, 2, &a_bytes) || !bytes_of(k, n, 2, &b_bytes) ||
      wgs > kaio::kMaxWorkgroups)
    return fail(KAIO_ERR_INVALID_PROBLEM, op, "problem too large for one launch (m=%u, n=%u, k=%u)", m, n, k);
  if (!c) return fail(KAIO_ERR_INVALID_ARGUMENT, op, "output c is null");
  if (k > 0 && !a) return fail(KAIO_ERR_INVALID_ARGUMENT, op, "input a is null");
  if (k > 0 && !b) return fail(KAIO_ERR_INVALID_ARGUMENT, op, "input b is null");
  if (!aligned16(c)) return fail(KAIO_ERR_INVALID_ARGUMENT, op, "output c is not 16-byte aligned");
  if (k > 0 && !aligned16(a)) return fail(KAIO_ERR_INVALID_ARGUMENT, op, "input a is not 16-byte aligned");
  if (k > 0 && !aligned16(b)) return fail(KAIO_ERR_INVALID_ARGUMENT, op, "input b is not 16-byte aligned");
  const Range ro[1] = {range(c, c_bytes, "c")};
  const Range ri[2] = {range(a, a_bytes, "a"), range(b, b_bytes, "b")};
  const Range* other = nullptr;
  if (const Range* o = overlap(ro, 1, ri, 2, &other))
    return fail(KAIO_ERR_INVALID_ARGUMENT, op, "output %s overlaps %s", o->name, other->name);
  if (kaio_status st = check_device(op)) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (k == 0) return launched(op, kaio::launch_fill_zero(c, c_bytes, s));
  return launched(op, kaio::launch_gemm_f16f32(static_cast<const uint16_t*>(a),
                                               static_cast<const uint16_t*>(b), c, m, n, k, s));
}

size_t kaio_gemm_f16f32_bwd_workspace_size(uint32_t m, uint32_t n) { return (size_t)m * n * 2; }

kaio_status kaio_gemm_f16f32_bwd(const void* a, const void* b, const float* grad, void* grad_a, void* grad_b,
                                 uint32_t m, uint32_t n, uint32_t k, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  return gemm_bwd("gemm_f16f32_bwd", a, b, grad, grad_a, grad_b, m, n, k, false, workspace, workspace_bytes,
                  stream);
}

kaio_status kaio_gemm_f16f32_bwd_noalloc(const void* a, const void* b, const float* grad, void* grad_a,
                                         void* grad_b, uint32_t m, uint32_t n, uint32_t k, void* stream) {
  return gemm_bwd("gemm_f16f32_bwd_noalloc", a, b, grad, grad_a, grad_b, m, n, k, true, nullptr, 0, stream);
}

kaio_status kaio_dequant_group_bwd(kaio_dtype dtype, int32_t outer, int32_t axis, int32_t group_size,
                                   const void* dy, const void* scale, void* dq, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  static const char* op = "dequant_group_bwd";
  (void)workspace;
  (void)workspace_bytes;
  // A C caller may pass any int here.  In C++ reading an enum object that holds a value
  // outside the enumeration's range is undefined, so the code is taken from the
  // parameter's bytes and only a validated code is turned back into a kaio_dtype.
  static_assert(sizeof(kaio_dtype) == sizeof(int), "kaio_dtype is passed as an int");
  int code = 0;
  std::memcpy(&code, &dtype, sizeof code);
  size_t esz = 0;
  switch (code) {
    case KAIO_DTYPE_F32: esz = 4; break;
    case KAIO_DTYPE_BF16: esz = 2; break;
    case KAIO_DTYPE_F16: esz = 2; break;
    case KAIO_DTYPE_F64: esz = 8; break;
    default:
      return fail(KAIO_ERR_UNSUPPORTED, op, "unsupported dtype %d (f32, bf16, f16, f64)", code);
  }
  const kaio_dtype dt = static_cast<kaio_dtype>(code);
  if (outer < 0 || axis < 0)
    return fail(KAIO_ERR_INVALID_PROBLEM, op, "outer_size (%d) and axis_size (%d) must be non-negative",
                outer, axis);
  if (group_size <= 0) return fail(KAIO_ERR_INVALID_PROBLEM, op, "group_size (%d) must be > 0", group_size);
  if (axis % group_size != 0)
    return fail(KAIO_ERR_INVALID_PROBLEM, op, "axis_size (%d) must be a multiple of group_size (%d)", axis,
                group_size);
  const uint64_t total = (uint64_t)outer * (uint64_t)axis;
  if (total == 0) return ok();
  uint64_t bytes = 0;
  if (!bytes_of(outer, axis, esz, &bytes))
    return fail(KAIO_ERR_INVALID_PROBLEM, op, "problem too large (outer=%d, axis=%d)", outer, axis);
  if (!dy) return fail(KAIO_ERR_INVALID_ARGUMENT, op, "d_output is null");
  if (!scale) return fail(KAIO_ERR_INVALID_ARGUMENT, op, "scale is null");
  if (!dq) return fail(KAIO_ERR_INVALID_ARGUMENT, op, "d_input is null");
  const void* ptrs[3] = {dy, scale, dq};
  static const char* names[3] = {"d_output", "scale", "d_input"};
  for (int i = 0; i < 3; ++i)
    if (reinterpret_cast<uintptr_t>(ptrs[i]) % esz != 0)
      return fail(KAIO_ERR_INVALID_ARGUMENT, op, "%s is not aligned to its element size (%zu)", names[i], esz);
  const Range ro[1] = {range(dq, bytes, "d_input")};
  const Range ri[2] = {range(dy, bytes, "d_output"),
                       range(scale, (uint64_t)outer * (uint64_t)(axis / group_size) * esz, "scale")};
  const Range* other = nullptr;
  if (const Range* o = overlap(ro, 1, ri, 2, &other))
    return fail(KAIO_ERR_INVALID_ARGUMENT, op, "output %s overlaps %s", o->name, other->name);
  if (kaio_status st = check_device(op)) return st;
  (void)hipGetLastError();
  return launched(op, kaio::launch_dequant_group_bwd(dt, outer, axis, group_size, dy, scale, dq,
                                                     static_cast<hipStream_t>(stream)));
}

kaio_status kaio_qkv_plan(uint32_t m, uint32_t n, uint32_t k, uint32_t bits, uint32_t plan[5]) {
  static const char* op = "qkv_plan";
  if (bits != 4 && bits != 8) return fail(KAIO_ERR_INVALID_ARGUMENT, op, "bits (%u) must be 4 or 8", bits);
  if (!plan) return fail(KAIO_ERR_INVALID_ARGUMENT, op, "plan is null");
  if (k % 128 != 0)
    return fail(KAIO_ERR_INVALID_PROBLEM, op, "K (%u) must be a multiple of group_size (128)", k);
  for (int i = 0; i < 5; ++i) plan[i] = 0;
  if (m == 0 || n == 0) return ok();
  if (kaio::qkv_split_k(m, k, bits)) {
    const uint32_t bn = kaio::decode_bn(m);
    plan[2] = bn;
    plan[3] = 1;
    plan[4] = (uint32_t)(3ull * ((n + bn - 1) / bn));
  } else {
    const kaio::PrefillForm f = kaio::tile_form(m, n, k, bits);
    plan[0] = f.outs == 1 ? 2 : 1;
    plan[1] = f.waves;
    plan[2] = f.bm;
    plan[3] = f.sets;
    const uint64_t wgs = kaio::prefill_wgs(f, m, n);
    plan[4] = wgs > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)wgs;
  }
  return ok();
}

const char* kaio_last_error(void) { return g_last_error.c_str(); }

const char* kaio_version(void) { return "kaio-mi355x 0.1.0 gfx950"; }

}  // extern "C"
