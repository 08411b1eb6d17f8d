// gdn_attention.hip -- the hybrid's gated full-attention mixer on gfx950.
//
// Every fourth layer of the hybrid is softmax attention with grouped queries
// ("Qwen3-Next 80B-A3B" field guide, cutaway 03: 16 query heads share 2 key/value
// heads, head dim 256; RoPE on the first 64 dims; QK-Norm; a learned sigmoid output
// gate.  "Qwen3.8-Flash-Next" model card, attention entries: per-head RMSNorm of q and
// k before RoPE, the rotate/nope split, attn_output * sigmoid(gate)):
//   q^ = RoPE(RMSNorm(q) w_q),  k^ = RoPE(RMSNorm(k) w_k)   (positions from 0 per sequence)
//   o  = softmax_causal(q^ k^T * scale) v * sigmoid(gate),  q head h -> kv head h / (Hq/Hkv)
//
// Two kernels:
//   qk_prep_kernel   one pass over q and k: RMSNorm, weight, rotate-half RoPE of the
//                    first rotary_dim dims (angles in fp64, reduced mod 2 pi before the
//                    fp32 sine and cosine) -> fp16 q^, k^ in the workspace;
//   attention_kernel one workgroup = 64 queries of one q head (4 waves x 16 queries),
//                    keys in tiles of 32 through LDS.  It computes S^T = K^ Q^T and
//                    O^T = V^T P^T on MFMA, so a query is a column of both: its lane
//                    holds its softmax statistics, and P^T (C layout of S^T) is already
//                    the B operand of the second product (k slots in the permuted
//                    order the A operand V^T reads).  Online softmax in base 2.
#include "gdn_attention.h"
#include "gdn_device.h"

#include <cmath>

namespace gdn {

// Set by a call whose cu_seqlens table is invalid; read and cleared by
// take_attention_error().
__device__ int g_attn_bad_cu = 0;

namespace {

typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;

constexpr int kAD = 256;          // head dim the kernels are built for
constexpr int kQB = 64;           // queries per workgroup
constexpr int kKT = 32;           // keys per tile
constexpr int kKsS = kAD + 8;     // fp16 row stride of the K^ tile [32 keys][256]
constexpr int kVtS = kKT + 8;     // bf16 row stride of the V^T tile [256][32 keys]

__device__ __forceinline__ f32x4 mfma_h(u16x8 a, u16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_b(u16x8 a, u16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// First token of the sequence holding token t (cu may be NULL: one sequence).
__device__ __forceinline__ int seq_begin(const int32_t *cu, int N, int t) {
  if (!cu) return 0;
  int lo = 0, hi = N;  // cu[lo] <= t < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid;
    else hi = mid;
  }
  return cu[lo];
}

// Max / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the lanes of one query).
__device__ __forceinline__ float rows4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows4_add(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// 256 threads = 8 rows of 256 (32 threads x 8 dims each); rows ordered token-major,
// q heads then kv heads.
__global__ void __launch_bounds__(256)
qk_prep_kernel(const bf16_t *__restrict__ q, const bf16_t *__restrict__ k,
               const int32_t *__restrict__ cu, int N, int T, int Hq, int Hkv,
               const float *__restrict__ wq, const float *__restrict__ wk, int rot,
               double log2_theta, float eps, int *__restrict__ bad_word,
               _Float16 *__restrict__ qh, _Float16 *__restrict__ kh) {
  if (blockIdx.x == 0 && bad_word) {
    // cu_seqlens check for this call: cu[0] = 0, non-decreasing, cu[N] = T
    int bad = 0;
    for (int i = threadIdx.x; i <= N; i += blockDim.x) {
      const int c = cu[i];
      if ((i == 0 && c != 0) || (i == N && c != T) || (i < N && cu[i + 1] < c)) bad = 1;
    }
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) {
      *bad_word = bad;
      if (bad) g_attn_bad_cu = 1;
    }
  }
  const int H = Hq + Hkv;
  const int64_t row = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
  const int j = threadIdx.x & 31;  // dims 8j .. 8j + 7
  if (row >= (int64_t)T * H) return;  // uniform per 32-lane row group
  const int t = (int)(row / H), hh = (int)(row % H);
  const bool isq = hh < Hq;
  const bf16_t *src = isq ? q + ((int64_t)t * Hq + hh) * kAD : k + ((int64_t)t * Hkv + hh - Hq) * kAD;
  const float *w = isq ? wq : wk;
  const uint4 raw = *reinterpret_cast<const uint4 *>(src + 8 * j);
  const uint32_t rw[4] = {raw.x, raw.y, raw.z, raw.w};
  float x[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = __uint_as_float(rw[e] << 16);
    x[2 * e + 1] = __uint_as_float(rw[e] & 0xFFFF0000u);
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 32);
  const float inv = rsqrtf(ss * (1.0f / kAD) + eps);
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = x[e] * inv * (w ? w[8 * j + e] : 1.0f);
  // rotate-half RoPE on dims < rot: dim d < rot/2 pairs with d + rot/2 (8-dim groups
  // rot/16 apart); every lane takes part in the exchange, only rotary lanes use it
  const int half = rot >> 1, sh = half >> 3;
  float pr[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int partner = (8 * j < half) ? j + sh : j - sh;
    pr[e] = __shfl(y[e], (int)(threadIdx.x & 32) + (partner & 31), 64);
  }
  if (8 * j < rot) {
    const int pos = t - seq_begin(cu, N, t);
    const bool lo = 8 * j < half;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = (lo ? 8 * j : 8 * j - half) + e;  // frequency index
      // angle pos * theta^(-2i/rot) in fp64, reduced to [-pi, pi] before sin/cos
      double ang = (double)pos * exp2(-2.0 * i / rot * log2_theta);
      ang -= 6.283185307179586 * rint(ang * 0.15915494309189535);
      float s, c;
      sincosf((float)ang, &s, &c);
      y[e] = lo ? y[e] * c - pr[e] * s : y[e] * c + pr[e] * s;
    }
  }
  _Float16 *dst = isq ? qh + ((int64_t)t * Hq + hh) * kAD : kh + ((int64_t)t * Hkv + hh - Hq) * kAD;
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  h8 out;
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = (_Float16)y[e];
  *reinterpret_cast<h8 *>(dst + 8 * j) = out;
}

__global__ void __launch_bounds__(256)
attention_kernel(const _Float16 *__restrict__ qh, const _Float16 *__restrict__ kh,
                 const bf16_t *__restrict__ v, const bf16_t *__restrict__ gate,
                 const int32_t *__restrict__ cu, int N, int T, int Hq, int Hkv, float scale2,
                 const int *__restrict__ bad_word, bf16_t *__restrict__ o) {
  __shared__ __attribute__((aligned(16))) _Float16 sK[kKT * kKsS];
  __shared__ __attribute__((aligned(16))) bf16_t sVt[kAD * kVtS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 15, lg = lane >> 4;
  // ids 8 apart go to the same XCD: the r = Hq/Hkv q heads of a kv head and query block
  // get ids 8 apart, so their shared K^ and V tiles are fetched into one L2
  const int r = Hq / Hkv;
  const int bid = blockIdx.x, x = bid & 7, yb = bid >> 3;
  const int member = yb % r, rest = (yb / r) * 8 + x;
  const int nqb = (T + kQB - 1) / kQB;
  if (rest >= nqb * Hkv) return;
  if (bad_word && *bad_word) return;  // invalid cu_seqlens: o is left unwritten
  // the last query blocks see the most keys: they are dispatched first
  const int qb = nqb - 1 - rest / Hkv, kvh = rest % Hkv;
  const int h = kvh * r + member;
  const int t0 = qb * kQB;
  const int tq = t0 + 16 * wave + ln;          // this lane's query
  const bool qvalid = tq < T;
  const int tqc = qvalid ? tq : T - 1;
  // its sequence's first token, and the first key any query of the block sees (both
  // clamped, so that no table can send an access out of bounds)
  const int sb = min(max(seq_begin(cu, N, tqc), 0), tqc);
  const int kstart = min(max(seq_begin(cu, N, t0), 0), t0);
  const int kend = min(t0 + kQB - 1, T - 1);   // last one

  // Q^ fragments (B operand of S^T = K^ Q^T): lane holds dims 32c + 8lg .. + 7 of its query
  u16x8 qf[8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
    qf[c] = *reinterpret_cast<const u16x8 *>(qh + ((int64_t)tqc * Hq + h) * kAD + 32 * c + 8 * lg);

  f32x4 oacc[16];
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  for (int k0 = kstart; k0 <= kend; k0 += kKT) {
    __syncthreads();  // the previous tile is consumed
    {  // K^ tile [32 keys][256]: thread = key tid / 8, dims 32 (tid % 8) .. + 31
      const int key = k0 + (tid >> 3), d0 = 32 * (tid & 7);
      uint4 w4[4] = {};
      if (key < T) {
        const uint4 *src = reinterpret_cast<const uint4 *>(kh + ((int64_t)key * Hkv + kvh) * kAD + d0);
#pragma unroll
        for (int i = 0; i < 4; ++i) w4[i] = src[i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint4 *>(sK + (tid >> 3) * kKsS + d0 + 8 * i) = w4[i];
    }
    {  // V^T tile [256][32 keys]: thread = keys 2 (tid % 16), + 1 and dims 16 (tid / 16) .. + 15
      const int kp = tid & 15, d0 = 16 * (tid >> 4);
      uint32_t a[8] = {}, b[8] = {};
      const int ka = k0 + 2 * kp, kb = ka + 1;
      if (ka < T) {
        const uint4 *s = reinterpret_cast<const uint4 *>(v + ((int64_t)ka * Hkv + kvh) * kAD + d0);
        const uint4 u0 = s[0], u1 = s[1];
        a[0] = u0.x; a[1] = u0.y; a[2] = u0.z; a[3] = u0.w; a[4] = u1.x; a[5] = u1.y; a[6] = u1.z; a[7] = u1.w;
      }
      if (kb < T) {
        const uint4 *s = reinterpret_cast<const uint4 *>(v + ((int64_t)kb * Hkv + kvh) * kAD + d0);
        const uint4 u0 = s[0], u1 = s[1];
        b[0] = u0.x; b[1] = u0.y; b[2] = u0.z; b[3] = u0.w; b[4] = u1.x; b[5] = u1.y; b[6] = u1.z; b[7] = u1.w;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {  // dims d0 + 2e (low halves) and d0 + 2e + 1 (high)
        *reinterpret_cast<uint32_t *>(sVt + (d0 + 2 * e) * kVtS + 2 * kp) =
            __builtin_amdgcn_perm(b[e], a[e], 0x05040100u);
        *reinterpret_cast<uint32_t *>(sVt + (d0 + 2 * e + 1) * kVtS + 2 * kp) =
            __builtin_amdgcn_perm(b[e], a[e], 0x07060302u);
      }
    }
    __syncthreads();

    // S^T [32 keys][16 queries] of this wave: two 16-key tiles
    f32x4 st[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      st[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const u16x8 a = *reinterpret_cast<const u16x8 *>(sK + (16 * kt + ln) * kKsS + 32 * c + 8 * lg);
        st[kt] = mfma_h(a, qf[c], st[kt]);
      }
    }
    // causal and sequence mask, base-2 logits, online softmax per query (lane column)
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = k0 + 16 * kt + 4 * lg + i;
        const bool ok = qvalid && key >= sb && key <= tq;
        st[kt][i] = ok ? st[kt][i] * scale2 : -INFINITY;
        mx = fmaxf(mx, st[kt][i]);
      }
    mx = rows4_max(mx);
    const float mn = fmaxf(m, mx);
    const float mu = mn == -INFINITY ? 0.f : mn;  // no key yet: every p is 0
    const float al = exp2f(m - mu);
    float ps = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        st[kt][i] = exp2f(st[kt][i] - mu);
        ps += st[kt][i];
      }
    l = l * al + rows4_add(ps);
    m = mn;
#pragma unroll
    for (int dt = 0; dt < 16; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[dt][i] *= al;
    // P^T as the B operand: slot 8lg + j <-> key 4lg + j (tile 0, j < 4), 16 + 4lg + j - 4
    const u16x8 pb = __builtin_bit_cast(
        u16x8, make_uint4(pk_bf16(st[0][0], st[0][1]), pk_bf16(st[0][2], st[0][3]),
                          pk_bf16(st[1][0], st[1][1]), pk_bf16(st[1][2], st[1][3])));
    // O^T += V^T P^T; V^T rows 16 dt + ln, keys in the same permuted order
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) {
      const bf16_t *row = sVt + (16 * dt + ln) * kVtS;
      const uint2 lo = *reinterpret_cast<const uint2 *>(row + 4 * lg);
      const uint2 hi = *reinterpret_cast<const uint2 *>(row + 16 + 4 * lg);
      const u16x8 a = __builtin_bit_cast(u16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
      oacc[dt] = mfma_b(a, pb, oacc[dt]);
    }
  }

  // epilogue: lane holds dims 16 dt + 4 lg .. + 3 of its query; o / l * sigmoid(gate)
  if (!qvalid) return;
  const float il = l > 0.f ? 1.0f / l : 0.f;
  const int64_t base = ((int64_t)tq * Hq + h) * kAD;
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) {
    const int d = 16 * dt + 4 * lg;
    const uint2 gw = *reinterpret_cast<const uint2 *>(gate + base + d);
    const float g[4] = {__uint_as_float(gw.x << 16), __uint_as_float(gw.x & 0xFFFF0000u),
                        __uint_as_float(gw.y << 16), __uint_as_float(gw.y & 0xFFFF0000u)};
    float val[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) val[i] = oacc[dt][i] * il * sigmoidf_(g[i]);
    *reinterpret_cast<uint2 *>(o + base + d) = make_uint2(pk_bf16(val[0], val[1]), pk_bf16(val[2], val[3]));
  }
}

}  // namespace

// Workspace: [256 B: this call's cu_seqlens verdict] [q^ fp16 T*Hq*256] [k^ fp16 T*Hkv*256]
size_t attention_workspace_bytes(int64_t T, int Hq, int Hkv) {
  if (T == 0) return 0;
  const size_t qb = ((size_t)T * Hq * kAD * 2 + 255) & ~(size_t)255;
  return 256 + qb + (size_t)T * Hkv * kAD * 2;
}

hipError_t take_attention_error(int *flag) {
  int zero = 0;
  hipError_t e = hipMemcpyFromSymbol(flag, HIP_SYMBOL(g_attn_bad_cu), sizeof(int));
  if (e != hipSuccess) return e;
  return *flag ? hipMemcpyToSymbol(HIP_SYMBOL(g_attn_bad_cu), &zero, sizeof(int)) : hipSuccess;
}

hipError_t launch_attention(const void *q, const void *k, const void *v, const void *gate,
                            const int32_t *cu, int N, int64_t T, int Hq, int Hkv,
                            const float *wq, const float *wk, int rotary_dim, float theta,
                            float eps, float scale, void *workspace, void *o,
                            hipStream_t stream) {
  if (T == 0) return hipSuccess;
  unsigned char *ws = (unsigned char *)workspace;
  int *bad_word = cu ? (int *)ws : nullptr;
  _Float16 *qh = (_Float16 *)(ws + 256);
  _Float16 *kh = (_Float16 *)(ws + 256 + (((size_t)T * Hq * kAD * 2 + 255) & ~(size_t)255));
  const int64_t rows = T * (Hq + Hkv);
  hipLaunchKernelGGL(qk_prep_kernel, dim3((unsigned)((rows + 7) / 8)), dim3(256), 0, stream,
                     (const bf16_t *)q, (const bf16_t *)k, cu, N, (int)T, Hq, Hkv, wq, wk,
                     rotary_dim, std::log2((double)theta), eps, bad_word, qh, kh);
  const int64_t nqb = (T + kQB - 1) / kQB;
  const int64_t pairs = nqb * Hkv;
  const int64_t blocks = (pairs + 7) / 8 * 8 * (Hq / Hkv);
  hipLaunchKernelGGL(attention_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const _Float16 *)qh, (const _Float16 *)kh, (const bf16_t *)v,
                     (const bf16_t *)gate, cu, N, (int)T, Hq, Hkv, scale * 1.4426950408889634f,
                     (const int *)bad_word, (bf16_t *)o);
  return hipGetLastError();
}

}  // namespace gdn
