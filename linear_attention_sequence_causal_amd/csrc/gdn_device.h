// gdn_device.h -- small device helpers shared by the gfx950 mixer kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr int kD = 128;     // head dim the kernels are built for
constexpr int kChunk = 64;  // tokens per chunk of the prefill

typedef uint16_t bf16_t;  // storage of a bf16 value
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) 16-byte load/store of fp32 data touched once.
__device__ __forceinline__ f32x4 ld_nt4(const float *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
}
__device__ __forceinline__ void st_nt4(float *p, f32x4 x) {
  __builtin_nontemporal_store(x, reinterpret_cast<f32x4 *>(p));
}

// fp32 -> bf16, round to nearest even (NaN stays NaN, Inf stays Inf).
__device__ __forceinline__ bf16_t f2bf(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}
__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

// hi = bf16(x), lo = bf16(x - hi): x = hi + lo to ~2^-16 relative.
__device__ __forceinline__ void split_bf(float x, bf16_t &hi, bf16_t &lo) {
  hi = f2bf(x);
  lo = f2bf(x - bf2f(hi));
}

template <typename T> struct Act;
template <> struct Act<float> {
  static __device__ __forceinline__ float load(const float *p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float *p, int64_t i, float x) { p[i] = x; }
};
template <> struct Act<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t *p, int64_t i) { return bf2f(p[i]); }
  static __device__ __forceinline__ void store(bf16_t *p, int64_t i, float x) { p[i] = f2bf(x); }
};

__device__ __forceinline__ float sigmoidf_(float u) { return 1.0f / (1.0f + __expf(-u)); }
__device__ __forceinline__ float siluf_(float u) { return u * sigmoidf_(u); }
// log(1 + e^u) without overflow: max(u, 0) + log1p(e^-|u|).
__device__ __forceinline__ float softplusf_(float u) {
  return fmaxf(u, 0.0f) + log1pf(__expf(-fabsf(u)));
}

// Log-decay g = -exp(A_log) * softplus(a + dt_bias), clamped below at -200 so
// that differences of chunk-local sums stay finite (exp(-200) is 0 in fp32).
__device__ __forceinline__ float log_decay(float a, float A_log, float dt_bias) {
  float g = -__expf(A_log) * softplusf_(a + dt_bias);
  return fmaxf(g, -200.0f);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
// Sum over lanes that differ only in bits below `width` (width a power of 2).
// (W <= 32; uses the LDS swizzle unit in bit-mask mode, lane ^ o within 32 lanes)
template <int PATTERN>
__device__ __forceinline__ float swizzle(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), PATTERN));
}
template <int W>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(W == 2 || W == 4 || W == 8 || W == 16 || W == 32, "group width");
  if (W >= 32) x += swizzle<0x1F | (16 << 10)>(x);
  if (W >= 16) x += swizzle<0x1F | (8 << 10)>(x);
  if (W >= 8) x += swizzle<0x1F | (4 << 10)>(x);
  if (W >= 4) x += swizzle<0x1F | (2 << 10)>(x);
  x += swizzle<0x1F | (1 << 10)>(x);
  return x;
}

// Value the optimiser cannot see through (keeps derived addresses local).
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

}  // namespace gdn
