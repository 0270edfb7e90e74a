// Shared device helpers of the gfx950 ClusterAttention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <string>

#define CA_DEV __device__ __forceinline__
#define CA_HD __host__ __device__ __forceinline__

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

namespace ca {

// ----------------------------------------------------------------------------
// Numbers
// ----------------------------------------------------------------------------

CA_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Round to nearest even; inputs here are finite.
CA_DEV uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

typedef float float2v_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));

// Two floats to packed bf16 (round to nearest even; v_cvt_pk_bf16_f32).
CA_DEV uint32_t pack_bf16x2(float lo, float hi) {
  const float2v_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2v_t));
}

// Element loads as float from a bf16 (uint16_t) or fp32 row.
CA_DEV float load_elem(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
CA_DEV float load_elem(const float* p, int64_t i) { return p[i]; }

// Monotone map of fp32 onto uint32 (a < b  <=>  key(a) < key(b)); -0 is
// treated as +0 so that values that compare equal get equal keys.
CA_DEV uint32_t order_key(float f) {
  if (f == 0.0f) f = 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ----------------------------------------------------------------------------
// splitmix64 (Steele, Lea & Flood, OOPSLA 2014): finaliser and streams.
// ----------------------------------------------------------------------------

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

CA_HD uint64_t fmix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// z <- fmix64((z ^ v) + golden) for each v, starting from z = 0.
CA_HD uint64_t chain_step(uint64_t z, uint64_t v) { return fmix64((z ^ v) + kGolden); }

constexpr uint64_t kDomainSample = 0x53;  // salt domain of the node subsample
constexpr uint64_t kDomainWarm = 0x57;    // salt domain of the warm-start vectors

// ----------------------------------------------------------------------------
// Tree layout: a node of n > c members splits at t = the multiple of c closest
// to n/2 with 1 <= t/c and t < n; equidistant -> the smaller (paper v1 §3.2.1).
// c is a power of two (64, 128 or 256).
// ----------------------------------------------------------------------------

CA_HD int split_size(int n, int c) {
  const int lc = __builtin_ctz((unsigned)c);   // c is a power of two
  int jmax = (n - 1) >> lc;
  int jl = n >> (lc + 1);
  int jh = jl + 1;
  if (jl < 1) jl = 1;
  if (jl > jmax) jl = jmax;
  if (jh < 1) jh = 1;
  if (jh > jmax) jh = jmax;
  long dl = 2L * jl * c - n; if (dl < 0) dl = -dl;
  long dh = 2L * jh * c - n; if (dh < 0) dh = -dh;
  return (dh < dl ? jh : jl) * c;
}

// Node in slot `idx` of depth `level`. Returns 1 and (off, n) if the node
// exists; 0 if an ancestor is already a leaf.
CA_HD int node_at(int N, int c, int level, int idx, int* off, int* n) {
  int o = 0, m = N;
  for (int l = 0; l < level; ++l) {
    if (m <= c) return 0;
    int t = split_size(m, c);
    if ((idx >> (level - 1 - l)) & 1) { o += t; m -= t; } else { m = t; }
  }
  *off = o;
  *n = m;
  return 1;
}

// The node of depth `level` that contains position p, or the leaf containing
// p if that leaf is shallower. Returns the depth reached.
CA_HD int node_of(int N, int c, int level, int p, int* off, int* n, int* idx) {
  int o = 0, m = N, j = 0, l = 0;
  for (; l < level; ++l) {
    if (m <= c) break;
    int t = split_size(m, c);
    if (p >= o + t) { o += t; m -= t; j = 2 * j + 1; } else { m = t; j = 2 * j; }
  }
  *off = o;
  *n = m;
  *idx = j;
  return l;
}

inline int tree_levels_host(int N, int c) {
  // depth of the deepest split + 1 (levels that contain a node of size > c)
  struct R {
    static int rec(int n, int c) {
      if (n <= c) return 0;
      int t = split_size(n, c);
      int a = rec(t, c), b = rec(n - t, c);
      return 1 + (a > b ? a : b);
    }
  };
  return R::rec(N, c);
}

// ----------------------------------------------------------------------------
// Wave helpers (wave64)
// ----------------------------------------------------------------------------

// Reductions over the two wave halves (lane l with lane l ^ 32), on the VALU:
// with both operands x, v_permlane32_swap leaves [x.lo, x.lo] in its first
// result and [x.hi, x.hi] in its second (lanes 0-31 | 32-63).
CA_DEV float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
CA_DEV float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

CA_DEV float wave_sum(float v) {
  v = sum_halves(v);
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

CA_DEV float wave_max(float v) {
  v = max_halves(v);
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

CA_DEV int lane_id() { return (int)(threadIdx.x & 63); }

// Exclusive prefix count of `flag` over the lanes below this one.
CA_DEV int lane_prefix(bool flag, uint64_t* total) {
  uint64_t b = __ballot(flag);
  *total = b;
  uint64_t below = (lane_id() == 0) ? 0ull : (b & (~0ull >> (64 - lane_id())));
  return __popcll(below);
}

}  // namespace ca

// ----------------------------------------------------------------------------
// Host-side error helpers
// ----------------------------------------------------------------------------

namespace ca {
void set_error(const std::string& s);
}

#define CA_HIP_CHECK(expr)                                                   \
  do {                                                                       \
    hipError_t e_ = (expr);                                                  \
    if (e_ != hipSuccess) {                                                  \
      ::ca::set_error(std::string(#expr) + ": " + hipGetErrorString(e_));    \
      return 4;                                                              \
    }                                                                        \
  } while (0)

// Raises a kernel's dynamic-LDS limit to `bytes` once per process (per call
// site; std::call_once makes the first launch from several host threads safe).
#define CA_MAX_LDS_ONCE(kernel_ptr, bytes)                                                 \
  do {                                                                                     \
    static std::once_flag once_;                                                           \
    std::call_once(once_, [&] {                                                            \
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel_ptr),                 \
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)(bytes)); \
    });                                                                                    \
  } while (0)
