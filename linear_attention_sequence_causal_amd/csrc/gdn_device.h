// gdn_device.h -- small device helpers shared by the gfx950 mixer kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr int kD = 128;     // head dim the kernels are built for
constexpr int kChunk = 32;  // tokens per chunk of the prefill

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
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(x));
}
__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }


template <typename T> struct Act;
template <> struct Act<float> {
  static __device__ __forceinline__ float load(const float *p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ uint32_t bits(const float *p, int64_t i) {
    return __float_as_uint(p[i]);
  }
  static __device__ __forceinline__ float from_bits(uint32_t b) { return __uint_as_float(b); }
  static __device__ __forceinline__ void store(float *p, int64_t i, float x) { p[i] = x; }
};
template <> struct Act<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t *p, int64_t i) { return bf2f(p[i]); }
  static __device__ __forceinline__ uint32_t bits(const bf16_t *p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ float from_bits(uint32_t b) { return __uint_as_float(b << 16); }
  static __device__ __forceinline__ void store(bf16_t *p, int64_t i, float x) { p[i] = f2bf(x); }
};

__device__ __forceinline__ float sigmoidf_(float u) { return 1.0f / (1.0f + __expf(-u)); }
// sigmoid with the hardware reciprocal (about 1 ulp) instead of an IEEE divide
__device__ __forceinline__ float sigmoid_fast(float u) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-u));
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// two fp32 -> packed bf16 pair (round to nearest even, one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
// two fp32 -> packed fp16 pair (round to nearest even, one v_cvt_pk_f16_f32)
__device__ __forceinline__ uint32_t pk_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, f16x2_t));
}
// hi/lo split of a pair: a = bf16(hi.x) + bf16(lo.x) to ~2^-16, same for b
__device__ __forceinline__ void split_pk(float a, float b, uint32_t &hi, uint32_t &lo) {
  hi = pk_bf16(a, b);
  const float ah = __uint_as_float(hi << 16), bh = __uint_as_float(hi & 0xFFFF0000u);
  lo = pk_bf16(a - ah, b - bh);
}
__device__ __forceinline__ float siluf_(float u) { return u * sigmoidf_(u); }
// Output gate of the epilogue: 0 SiLU(z), 1 sigmoid(z) (gdn_params.output_gate).
__device__ __forceinline__ float out_gate(int gate, float z) {
  const float s = sigmoidf_(z);
  return gate == 1 ? s : z * s;
}
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

// Log-decay with the hardware log/exp (absolute error ~1e-7 in softplus).
__device__ __forceinline__ float log_decay_fast(float a, float A_log, float dt_bias) {
  const float u = a + dt_bias;
  const float sp = fmaxf(u, 0.0f) + __logf(1.0f + __expf(-fabsf(u)));
  return fmaxf(-__expf(A_log) * sp, -200.0f);
}

// Inclusive prefix sum over the 64 lanes of a wave: shift-and-add inside each
// row of 16 lanes on the DPP crossbar, then the row totals via readlane.
__device__ __forceinline__ float wave_inclusive_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xF, 0xF, true));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 15));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 31));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 47));
  const int row = (threadIdx.x & 63) >> 4;
  if (row >= 1) x += r0;
  if (row >= 2) x += r1;
  if (row >= 3) x += r2;
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
// Sum over each row of 16 lanes (lanes 16r .. 16r+15), result in every lane of
// the row: a rotate-and-add butterfly on the DPP crossbar (no LDS traffic).
__device__ __forceinline__ float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false));
  return x;
}

// Maximum over the 64 lanes of a wave, left in every lane: a rotate-and-max
// butterfly inside each row of 16 lanes on the DPP crossbar, then the four row
// results via readlane.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false)));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// The same for x >= 0 (or NaN with the sign bit clear), returned uniform: such
// floats order like their bit patterns as unsigned integers, so the butterfly is
// an integer max that fuses with its DPP move, and the four row results are
// combined on the scalar unit.  A NaN comes out as a NaN.
__device__ __forceinline__ float wave_max_nonneg(float x) {
  uint32_t v = __float_as_uint(x);
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xF, 0xF, false));
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return __uint_as_float(max(max(r0, r1), max(r2, r3)));
}

// 1/sqrt(x) for x >= 0 as the bare v_rsq_f32: x is raised to the smallest normal
// float first (v_rsq_f32 takes no denormal input), so 0 gives 2^63, not infinity.
__device__ __forceinline__ float rsq_normal(float x) {
  return __builtin_amdgcn_rsqf(fmaxf(x, 1.17549435e-38f));
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Value the optimiser cannot see through (keeps derived addresses local).
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

}  // namespace gdn
