// gdn_decode.hip -- single-token decode step of the Gated DeltaNet mixer, gfx950.
//
// One workgroup per (sequence b, q/k head g) handles all r = Hv/Hk v heads that
// read g (the field guide's 16 q/k : 32 v head sharing), so it exclusively owns
// the conv-state channels of q/k head g and of those v heads and shifts them in
// place.  Work per workgroup:
//   1. conv (width 4: the 3 cached raw rows + the new row) + SiLU on the
//      channels of q, k and the r v heads; L2-normalise q and k; k.q.
//   2. per v head: gates alpha = exp(-exp(A_log) softplus(a + dt_bias)),
//      beta = sigmoid(b) (model card gated-DeltaNet entry; Fig. 2 caption).
//   3. stream the fp32 state H = S^T ([dk][dv]) once: the field guide's six
//      update steps fused into one read and one write,
//        vhat_j = alpha sum_i H_ij k_i                 (S' k)
//        e_j    = v_j - vhat_j
//        H_ij  <- alpha H_ij + beta k_i e_j             (S'' = S' + beta e k^T)
//        y_j    = alpha sum_i H_ij q_i + beta (k.q) e_j  (S'' q)
//   4. gated RMSNorm epilogue o = y rsqrt(mean y^2 + eps) w SiLU(z).
// The state is ~97% of the bytes moved, so the kernel is HBM-bound.  Each
// thread holds 64 floats of one head's state and already has the next head's
// 64 floats in flight while it works on the current one.
#include "gdn_device.h"

namespace gdn {

constexpr int kDecThreads = 256;
// stored state formats of the decode step
constexpr int kStateF32 = 0, kStateBf16 = 1, kStateFp8 = 2;
constexpr int kDecMaxRatio = 8;  // largest Hv / Hk the decode kernel accepts

// Stored state: fp32, or bf16 (rounded to nearest even on every store), or fp8 with
// one scale per row; the step itself is computed in fp32.  C consecutive columns of a
// row per access (16 bytes for fp32 and fp8, 8 for bf16), streamed once (non-temporal).
// A prefetched head is kept in its stored form (Raw) until it is used, so the narrow
// formats need fewer registers for it.
template <typename S> struct StateIO;
template <> struct StateIO<float> {
  static constexpr int C = 4;
  typedef f32x4 Raw;
  static __device__ __forceinline__ Raw load_raw(const float *p) { return ld_nt4(p); }
  static __device__ __forceinline__ void widen(Raw x, float (&o)[C]) {
    o[0] = x.x; o[1] = x.y; o[2] = x.z; o[3] = x.w;
  }
  static __device__ __forceinline__ void store(float *p, const float (&x)[C]) {
    st_nt4(p, f32x4{x[0], x[1], x[2], x[3]});
  }
};
template <> struct StateIO<bf16_t> {
  static constexpr int C = 4;
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  typedef u32x2 Raw;
  static __device__ __forceinline__ Raw load_raw(const bf16_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
  }
  static __device__ __forceinline__ void widen(Raw w, float (&o)[C]) {
    o[0] = __uint_as_float(w.x << 16); o[1] = __uint_as_float(w.x & 0xFFFF0000u);
    o[2] = __uint_as_float(w.y << 16); o[3] = __uint_as_float(w.y & 0xFFFF0000u);
  }
  static __device__ __forceinline__ void store(bf16_t *p, const float (&x)[C]) {
    const u32x2 w = {pk_bf16(x[0], x[1]), pk_bf16(x[2], x[3])};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2 *>(p));
  }
};

// fp8 storage: OCP E4M3 bytes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
// largest finite value 448) times one power-of-two scale per state row (dk index)
// kept in fp32 beside the state; the step's arithmetic is fp32.  16 columns per access.
struct fp8_t {
  uint8_t bits;
};
template <> struct StateIO<fp8_t> {
  static constexpr int C = 16;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef u32x4 Raw;
  static __device__ __forceinline__ Raw load_raw(const fp8_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  }
  // codes times the row scale sc (a power of two): one scaled conversion per 2 values
  static __device__ __forceinline__ void widen(Raw w, float sc, float (&o)[C]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const auto lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)w[q], sc, false);  // bytes 0, 1
      const auto hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)w[q], sc, true);   // bytes 2, 3
      o[4 * q] = lo[0]; o[4 * q + 1] = lo[1]; o[4 * q + 2] = hi[0]; o[4 * q + 3] = hi[1];
    }
  }
  // codes of x / sc for the row scale sc (a power of two, so the division is exact and
  // |x / sc| <= 448), rounded to nearest even
  static __device__ __forceinline__ void store(fp8_t *p, const float (&x)[C], float sc) {
    typedef short s16x2 __attribute__((ext_vector_type(2)));
    u32x4 w;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      s16x2 t = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32((s16x2){0, 0}, x[4 * q], x[4 * q + 1], sc,
                                                         false);
      t = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(t, x[4 * q + 2], x[4 * q + 3], sc, true);
      w[q] = __builtin_bit_cast(uint32_t, t);
    }
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(p));
  }
};

// Maximum over each group of 8 lanes (8g .. 8g+7), left in every lane of the group:
// swaps of neighbours and of pairs inside each quad, then the two quads of the group
// (row_half_mirror pairs lane i with 7 - i).
__device__ __forceinline__ float max8(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));   // quad_perm 1,0,3,2
  x = fmaxf(x, dpp_f<0x4E>(x));   // quad_perm 2,3,0,1
  return fmaxf(x, dpp_f<0x141>(x));  // row_half_mirror
}

// Exponent e of the fp8 row scale 2^e: the smallest with m <= 448 * 2^e, for a finite
// normal m > 0 (m = f 2^E, 1 <= f < 2: e = E - 8, or E - 7 when f > 1.75); 0 (scale 1)
// for zero, subnormal or non-finite m.
__device__ __forceinline__ int fp8_scale_exp(float m) {
  const uint32_t b = __float_as_uint(m);
  const int eb = (int)((b >> 23) & 0xFF);
  if (eb == 0 || eb == 255) return 0;
  const int e = eb - 127 - 8 + ((b & 0x7FFFFF) > 0x600000u ? 1 : 0);
  return min(max(e, -126), 127);
}

// Sum of x over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the 16-lane rows of a
// wave), left in all four: two row swaps on the gfx950 permlane crossbar.
__device__ __forceinline__ float rows4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// Sum over the 64 lanes, left in every lane: a DPP sum inside each 16-lane row, then
// the four rows (about 8 instructions, against ~30 for a shuffle butterfly).
__device__ __forceinline__ float wave_sum_dpp(float x) { return rows4_sum(row16_sum(x)); }
// SiLU with the hardware reciprocal (about 1 ulp) instead of an IEEE divide
__device__ __forceinline__ float silu_fast(float u) { return u * sigmoid_fast(u); }

template <typename T, typename S>
__global__ void __launch_bounds__(kDecThreads)
decode_step_kernel(const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
                   const float *__restrict__ a, const float *__restrict__ b,
                   const T *__restrict__ z, const float *__restrict__ conv_w,
                   const float *__restrict__ A_log, const float *__restrict__ dt_bias,
                   const float *__restrict__ norm_w, float q_scale, float l2_eps, float rms_eps,
                   S *__restrict__ state, float *__restrict__ state_scale,
                   T *__restrict__ conv_state, T *__restrict__ o, int Hk, int Hv, int gate) {
  constexpr bool kFp8 = __is_same(S, fp8_t);
  const int g = blockIdx.x % Hk;
  const int bseq = blockIdx.x / Hk;
  const int r = Hv / Hk;
  const int tid = threadIdx.x;
  const int64_t Cc = 2LL * Hk * kD + (int64_t)Hv * kD;

  // thread t of the state stream: columns CPT*(t%NCG)..+CPT-1 of rows RPT*(t/NCG)..+RPT-1
  // (fp32 and bf16: 4 columns of 16 rows; fp8: 16 columns of 4 rows, i.e. 16-byte
  // accesses and a row's scale from a max over 8 lanes)
  constexpr int CPT = StateIO<S>::C;
  constexpr int NCG = kD / CPT;            // threads per state row
  constexpr int NRG = kDecThreads / NCG;   // row groups
  constexpr int RPT = kD / NRG;            // rows per thread
  static_assert(RPT % 4 == 0 && (!kFp8 || NCG == 8), "state stream layout");

  __shared__ float s_x[2 + kDecMaxRatio][kD];  // post-prologue q, k, then v of each v head
  // partial column sums: per row group (fp32, bf16), or per wave once each wave has
  // summed its own eight row groups on the crossbar (fp8)
  constexpr int NRED = kFp8 ? kDecThreads / 64 : NRG;
  __shared__ float s_red[NRED][2][kD];
  __shared__ float s_e[kD];
  __shared__ float s_y[kD];
  __shared__ float s_misc[4];

  const int col = (tid % NCG) * CPT;
  const int rg = tid / NCG;
  const int row0 = rg * RPT;
  auto head_ptr = [&](int j) {
    return state + (((int64_t)bseq * Hv + r * g + j) * kD + row0) * kD + col;
  };
  // Small inputs go out before the state: vector-memory waits are in issue order,
  // so a wait for one of them never queues behind a state prefetch.
  // (unconditional, as bit patterns widened at first use: a conditional load would be
  // widened, and waited for, before the state loads are issued; threads >= kD read a
  // valid element and ignore it)
  const int ztid = tid & (kD - 1);
  const float nwv = norm_w ? norm_w[ztid] : 1.0f;
  uint32_t zbits = Act<T>::bits(z, ((int64_t)bseq * Hv + r * g) * kD + ztid);
  // Start streaming the first head's state before the prologue.
  typename StateIO<S>::Raw Hraw[RPT];
  f32x4 Sraw[RPT / 4];  // fp8 storage: the scales of this thread's rows
  auto scale_ptr = [&](int j) {
    return state_scale + ((int64_t)bseq * Hv + r * g + j) * kD + row0;
  };
  {
    const S *Hp = head_ptr(0);
#pragma unroll
    for (int i = 0; i < RPT; ++i) Hraw[i] = StateIO<S>::load_raw(Hp + i * kD);
    if (kFp8) {
#pragma unroll
      for (int i = 0; i < RPT / 4; ++i) Sraw[i] = *reinterpret_cast<const f32x4 *>(scale_ptr(0) + 4 * i);
    }
  }

  // ---- 1. prologue --------------------------------------------------------------
  // Pass 0: sections (64 threads each) = q, k, v of heads 0 and 1 of the group;
  // pass p >= 1: v heads 2 + 4(p-1) + section.  Each thread takes 2 channels.
  T *cs = conv_state + (int64_t)bseq * 3 * Cc;
  const int c0 = (tid & 63) * 2;
  const int sec = tid >> 6;
  for (int pass = 0; pass == 0 || 2 + 4 * (pass - 1) < r; ++pass) {
    int slot, jv = -1;
    if (pass == 0) {
      slot = sec;
      if (sec >= 2) jv = sec - 2;
    } else {
      jv = 2 + 4 * (pass - 1) + sec;
      slot = 2 + jv;
    }
    const bool active = jv < r;  // jv = -1 for q and k
    int64_t cbase;
    const T *src;
    int64_t sidx;
    if (slot == 0) {
      cbase = (int64_t)g * kD;
      src = q;
      sidx = ((int64_t)bseq * Hk + g) * kD;
    } else if (slot == 1) {
      cbase = (int64_t)Hk * kD + (int64_t)g * kD;
      src = k;
      sidx = ((int64_t)bseq * Hk + g) * kD;
    } else {
      cbase = 2LL * Hk * kD + (int64_t)(r * g + jv) * kD;
      src = v;
      sidx = ((int64_t)bseq * Hv + r * g + jv) * kD;
    }
    float xv[2] = {0.f, 0.f};
    if (active) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int64_t ch = cbase + c0 + u;
        const float raw = Act<T>::load(src, sidx + c0 + u);
        const float h0 = Act<T>::load(cs, ch), h1 = Act<T>::load(cs, Cc + ch),
                    h2 = Act<T>::load(cs, 2 * Cc + ch);
        const float4 w = *reinterpret_cast<const float4 *>(conv_w + ch * 4);
        xv[u] = silu_fast(w.x * h0 + w.y * h1 + w.z * h2 + w.w * raw);
        // shift the cache in place (reads above precede these writes)
        Act<T>::store(cs, ch, h1);
        Act<T>::store(cs, Cc + ch, h2);
        Act<T>::store(cs, 2 * Cc + ch, raw);
      }
    }
    if (slot < 2) {  // L2-normalise q (wave 0) and k (wave 1) over 128 channels
      const float ss = wave_sum_dpp(xv[0] * xv[0] + xv[1] * xv[1]);
      const float f = (slot == 0 ? q_scale : 1.0f) * rsq_normal(ss + l2_eps);
      xv[0] *= f;
      xv[1] *= f;
    }
    if (active) {
      s_x[slot][c0] = xv[0];
      s_x[slot][c0 + 1] = xv[1];
    }
  }
  __syncthreads();
  if (tid < 64) {
    const float kq = wave_sum_dpp(s_x[0][2 * tid] * s_x[1][2 * tid] +
                              s_x[0][2 * tid + 1] * s_x[1][2 * tid + 1]);
    if (tid == 0) s_misc[0] = kq;
  }
  __syncthreads();
  const float kq = s_misc[0];

  float kr[RPT], qr[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    kr[i] = s_x[1][row0 + i];
    qr[i] = s_x[0][row0 + i];
  }

  // ---- 3./4. per v head: state stream and epilogue ---------------------------------
  for (int j = 0; j < r; ++j) {
    const int h = r * g + j;
    const float zv = Act<T>::from_bits(zbits), sz = sigmoid_fast(zv);
    const float zg = gate == 1 ? sz : zv * sz;  // output gate sigmoid(z) or SiLU(z)
    if (j + 1 < r) zbits = Act<T>::bits(z, ((int64_t)bseq * Hv + h + 1) * kD + ztid);
    // the next head's loads go out first (vector-memory waits are in issue order, so
    // waiting for this head's state does not wait for them)
    typename StateIO<S>::Raw Hnext[RPT];
    f32x4 Snext[RPT / 4];
    if (j + 1 < r) {
      const S *Hn = head_ptr(j + 1);
#pragma unroll
      for (int i = 0; i < RPT; ++i) Hnext[i] = StateIO<S>::load_raw(Hn + i * kD);
      if (kFp8) {
#pragma unroll
        for (int i = 0; i < RPT / 4; ++i)
          Snext[i] = *reinterpret_cast<const f32x4 *>(scale_ptr(j + 1) + 4 * i);
      }
    }
    // fp32 / bf16: the head widened once (64 fp32 registers).  fp8: each row widened where
    // it is used (twice), which keeps the workgroup under 128 VGPRs (four per compute
    // unit, more state bytes in flight); the raw words pass an optimisation barrier
    // before the second widening so that it is not merged with the first.
    float Hcur[kFp8 ? 1 : RPT][CPT];
    if constexpr (!kFp8) {
#pragma unroll
      for (int i = 0; i < RPT; ++i) StateIO<S>::widen(Hraw[i], Hcur[i]);
    }
    auto row = [&](int i, float (&t)[CPT]) __attribute__((always_inline)) {
      if constexpr (kFp8) StateIO<S>::widen(Hraw[i], Sraw[i >> 2][i & 3], t);
      else {
#pragma unroll
        for (int c = 0; c < CPT; ++c) t[c] = Hcur[i][c];
      }
    };
    const float alpha = __expf(log_decay(a[(int64_t)bseq * Hv + h], A_log[h], dt_bias[h]));
    const float beta = sigmoid_fast(b[(int64_t)bseq * Hv + h]);
    float sk[CPT], sq[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) sk[c] = sq[c] = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      float t[CPT];
      row(i, t);
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        sk[c] += t[c] * kr[i];
        sq[c] += t[c] * qr[i];
      }
    }
    if constexpr (kFp8) {
      // The wave's eight row groups are lane bits 3-5 (lane = 8 x row group + column
      // group).  Reduce-scatter over them: each step pairs two value sets, and the lanes
      // with the step's bit clear keep the first set summed over the lane pair, those
      // with it set the second.  After the three steps lane (b5, b4, b3) holds values
      // 16 b5 + 8 b4 + 4 b3 + 0..3 of the 32 (sk, then sq), summed over the wave.
      float w16[16], w8[8], w4[4];
#pragma unroll
      for (int m = 0; m < 16; ++m) {  // bit 5: sk for the lower half, sq for the upper
        const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(sk[m]),
                                                        __float_as_uint(sq[m]), false, false);
        w16[m] = __uint_as_float(t[0]) + __uint_as_float(t[1]);
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) {  // bit 4: the 16-lane rows
        const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(w16[m]),
                                                        __float_as_uint(w16[m + 8]), false, false);
        w8[m] = __uint_as_float(t[0]) + __uint_as_float(t[1]);
      }
      const bool b3 = (tid & 8) != 0;
#pragma unroll
      for (int m = 0; m < 4; ++m) {  // bit 3: lane l and l ^ 8 (rotate by 8 in a row)
        const float send = b3 ? w8[m] : w8[m + 4];
        const float keep = b3 ? w8[m + 4] : w8[m];
        w4[m] = keep + dpp_f<0x128>(send);
      }
      const int lane = tid & 63;
      *reinterpret_cast<f32x4 *>(&s_red[tid >> 6][lane >> 5][col + (lane & 0x18) / 2]) =
          f32x4{w4[0], w4[1], w4[2], w4[3]};
    } else {
#pragma unroll
      for (int c = 0; c < CPT; c += 4) {
        *reinterpret_cast<f32x4 *>(&s_red[rg][0][col + c]) = f32x4{sk[c], sk[c + 1], sk[c + 2], sk[c + 3]};
        *reinterpret_cast<f32x4 *>(&s_red[rg][1][col + c]) = f32x4{sq[c], sq[c + 1], sq[c + 2], sq[c + 3]};
      }
    }
    __syncthreads();
    if (tid < kD) {
      float vk = 0.f, vq = 0.f;
#pragma unroll
      for (int p = 0; p < NRED; ++p) {
        vk += s_red[p][0][tid];
        vq += s_red[p][1][tid];
      }
      const float e = s_x[2 + j][tid] - alpha * vk;  // e = v - S'k
      const float y = alpha * vq + beta * kq * e;    // S'' q
      s_e[tid] = e;
      s_y[tid] = y;
      const float ssum = wave_sum_dpp(y * y);
      if ((tid & 63) == 0) s_misc[1 + (tid >> 6)] = ssum;
    }
    __syncthreads();
    float ec[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) ec[c] = beta * s_e[col + c];
    S *Hp = head_ptr(j);
    float snew[RPT];  // fp8 storage: the new row scales
    if constexpr (kFp8) {
#pragma unroll
      for (int i = 0; i < RPT; ++i)
#pragma unroll
        for (int w = 0; w < 4; ++w) asm volatile("" : "+v"(Hraw[i][w]));
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      float hn[CPT];
      row(i, hn);
#pragma unroll
      for (int c = 0; c < CPT; ++c) hn[c] = alpha * hn[c] + kr[i] * ec[c];
      if constexpr (kFp8) {  // the row's scale: max over its 128 columns (8 lanes x 16)
        float m = fabsf(hn[0]);
#pragma unroll
        for (int c = 1; c < CPT; ++c) m = fmaxf(m, fabsf(hn[c]));
        const int e = fp8_scale_exp(max8(m));
        snew[i] = __uint_as_float((uint32_t)(127 + e) << 23);  // 2^e, e in [-126, 127]
        StateIO<S>::store(Hp + i * kD, hn, snew[i]);
      } else {
        StateIO<S>::store(Hp + i * kD, hn);
      }
    }
    if (kFp8 && (tid % NCG) == 0) {
#pragma unroll
      for (int i = 0; i < RPT; i += 4)
        *reinterpret_cast<f32x4 *>(scale_ptr(j) + i) = f32x4{snew[i], snew[i + 1], snew[i + 2], snew[i + 3]};
    }
    if (tid < kD) {
      const float inv = rsq_normal((s_misc[1] + s_misc[2]) * (1.0f / kD) + rms_eps);
      Act<T>::store(o, ((int64_t)bseq * Hv + h) * kD + tid, s_y[tid] * inv * nwv * zg);
    }
    __syncthreads();  // s_red, s_e, s_y, s_misc are reused by the next head
    if (j + 1 < r) {
#pragma unroll
      for (int i = 0; i < RPT; ++i) Hraw[i] = Hnext[i];
      if (kFp8) {
#pragma unroll
        for (int i = 0; i < RPT / 4; ++i) Sraw[i] = Snext[i];
      }
    }
  }
}

// state_bf16: the state is bf16 storage (void * either way)
template <typename T>
hipError_t launch_decode(const void *q, const void *k, const void *v, const float *a,
                         const float *b, const void *z, const float *conv_w, const float *A_log,
                         const float *dt_bias, const float *norm_w, float q_scale, float l2_eps,
                         float rms_eps, void *state, int state_kind, float *state_scale,
                         void *conv_state, void *o, int batch, int Hk, int Hv, int gate,
                         hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  dim3 grid((unsigned)batch * (unsigned)Hk);
  auto go = [&](auto kern, auto *st) {
    hipLaunchKernelGGL(kern, grid, dim3(kDecThreads), 0, stream, (const T *)q, (const T *)k,
                       (const T *)v, a, b, (const T *)z, conv_w, A_log, dt_bias, norm_w, q_scale,
                       l2_eps, rms_eps, st, state_scale, (T *)conv_state, (T *)o, Hk, Hv,
                       gate);
  };
  if (state_kind == kStateBf16) go(decode_step_kernel<T, bf16_t>, (bf16_t *)state);
  else if (state_kind == kStateFp8) go(decode_step_kernel<T, fp8_t>, (fp8_t *)state);
  else go(decode_step_kernel<T, float>, (float *)state);
  return hipGetLastError();
}

int decode_max_ratio() { return kDecMaxRatio; }

template hipError_t launch_decode<float>(const void *, const void *, const void *, const float *,
                                         const float *, const void *, const float *,
                                         const float *, const float *, const float *, float,
                                         float, float, void *, int, float *, void *, void *, int,
                                         int, int, int, hipStream_t);
template hipError_t launch_decode<bf16_t>(const void *, const void *, const void *,
                                          const float *, const float *, const void *,
                                          const float *, const float *, const float *,
                                          const float *, float, float, float, void *, int,
                                          float *, void *, void *, int, int, int, int,
                                          hipStream_t);

// ---------------------------------------------------------------------------------
// Multi-token step: n (1..8) new tokens per sequence on a cached state.  It is the
// single step above applied to the tokens in order (per token the field guide's
// six update operations, cutaway 02, and the same gates and epilogue), but each
// fp32 state is read once and written at most once for all n tokens, so the bytes
// per token drop n-fold.  Token t's output sees tokens 0..t.  The state and the
// conv cache advance by commit = num_commit[b] tokens (clamped to 0..n; n when
// num_commit is NULL): the state is written right after token commit - 1 and not
// at all when commit = 0.  A speculative verify pass (commit 0) thus leaves both
// untouched, and a second pass with the accepted count advances them.
constexpr int kMaxStepTokens = 8;


// One workgroup of four waves per (sequence, v head), in the chunk form of the n
// tokens: with Gam_t the decay product of tokens 0..t and R_ts = Gam_t / Gam_s (the
// product of the decays of tokens s+1..t), unrolling the per-token update gives
//   u_t = beta_t (v_t - Gam_t S_0 k_t - sum_{s<t} R_ts (k_s . k_t) u_s),
//   y_t = Gam_t S_0 q_t + sum_{s<=t} R_ts (k_s . q_t) u_s,
//   S_c = Gam_{c-1} S_0 + sum_{s<c} R_{c-1,s} u_s k_s^T     (after c tokens),
// so every state product is taken against the state the call starts from, S_0:
// the products S_0 k_t and S_0 q_t of all n tokens, then per value column an n x n
// triangular recurrence, then one rank-c update.  Both products run on fp32 MFMA
// (4x4x1 with the A operand broadcast to the 16 blocks, i.e. an outer product of
// four values with the 64 lanes), with the state in the accumulator layout:
// wave w holds key rows 64 (w & 1) .. + 63 and value columns 64 (w >> 1) .. + 63,
// register i of tile m = row 4 m + i of that range, lane = value column.  As the B
// operand of the first product each register is one key row; as the accumulator of
// the update, one MFMA per tile adds a token's rank-1 term.  The two key-row halves'
// partial products meet in LDS.  The r workgroups of a q/k head each convolve its q
// and k rows from the cache and only read the cache's q/k channels; a second
// kernel on the same stream advances those channels after every workgroup has read
// them (qk_cache_advance_kernel), so no workgroup reads a cache word that another
// one of the same launch writes.  The v channels of a head are read and advanced by
// the thread that convolves them, in its head's workgroup.
constexpr int kTokThreads = 256;
// One v head's fp32 state as a raw buffer: each lane's words are addressed by its
// own offset plus a uniform row offset, so no per-row 64-bit addresses are kept in
// registers.  Cache policy non-temporal (the state is touched once per call).
constexpr int kNtPolicy = 2;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t state_buf(float *base) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, kD * kD * (int)sizeof(float),
                                           0x00020000);
}
__device__ __forceinline__ float ld_row1(__amdgpu_buffer_rsrc_t r, uint32_t off, int row_off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, row_off, kNtPolicy));
}
__device__ __forceinline__ void st_row1(__amdgpu_buffer_rsrc_t r, uint32_t off, int row_off,
                                        float x) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, off, row_off, kNtPolicy);
}
// C[i][lane] += a[4 abid + i] * b[lane] (i = 0..3): the four values of block abid
// of a broadcast to all 16 blocks of the 4x4x1 fp32 product.
template <int ABID>
__device__ __forceinline__ f32x4 outer4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_4x4x1f32(a, b, c, 4, ABID, 0);
}

// The four key rows of one state tile (its registers 0..3) against blocks B0 .. B0 + 3
// of the k and q operands.
template <int B0>
__device__ __forceinline__ void rows4(float ak, float aq, f32x4 hm, f32x4 &yk, f32x4 &yq) {
  yk = outer4<B0>(ak, hm[0], yk);     yq = outer4<B0>(aq, hm[0], yq);
  yk = outer4<B0 + 1>(ak, hm[1], yk); yq = outer4<B0 + 1>(aq, hm[1], yq);
  yk = outer4<B0 + 2>(ak, hm[2], yk); yq = outer4<B0 + 2>(aq, hm[2], yq);
  yk = outer4<B0 + 3>(ak, hm[3], yk); yq = outer4<B0 + 3>(aq, hm[3], yq);
}

// NG groups of four token slots (n <= 4 NG).
template <typename T, int NG>
__global__ void __launch_bounds__(kTokThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
decode_tokens_kernel(const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
                     const float *__restrict__ a, const float *__restrict__ b,
                     const T *__restrict__ z, const float *__restrict__ conv_w,
                     const float *__restrict__ A_log, const float *__restrict__ dt_bias,
                     const float *__restrict__ norm_w, float q_scale, float l2_eps,
                     float rms_eps, float *__restrict__ state, T *__restrict__ conv_state,
                     const int32_t *__restrict__ num_commit, T *__restrict__ o, int Hk, int Hv,
                     int n, int gate) {
  constexpr int NT = 4 * NG;  // token slots
  const int r = Hv / Hk;
  const int jh = blockIdx.x % r;                  // v head within its q/k group
  const int g = (blockIdx.x / r) % Hk;            // q/k head
  const int bseq = blockIdx.x / r / Hk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t Cc = 2LL * Hk * kD + (int64_t)Hv * kD;
  const int commit = num_commit ? min(max(num_commit[bseq], 0), n) : n;

  // v head (the clamp is a no-op; in this form the kernel fits 128 registers unspilled)
  const int h = r * g + min(jh, r - 1);
  const int dh = wave & 1, chh = wave >> 1;
  const int d0 = 64 * dh;                         // key rows d0 .. d0 + 63
  const int col = 64 * chh + lane;                // this lane's value column

  __shared__ float s_x[kMaxStepTokens][3][kD];    // post-prologue q, k, v rows
  __shared__ f32x4 s_yp[2][2][2 * NG][64];        // [key half][column half][k|q, group]
  __shared__ float s_ab[kMaxStepTokens][2];       // alpha, beta of each token
  __shared__ float s_cq[kMaxStepTokens][kMaxStepTokens];  // R_ts (k_s . q_t), s <= t
  __shared__ float s_ck[kMaxStepTokens][kMaxStepTokens];  // R_ts (k_s . k_t), s < t
  __shared__ float s_R[kMaxStepTokens][kMaxStepTokens];   // R_ts
  __shared__ float s_G[kMaxStepTokens];                   // Gam_t
  __shared__ float s_ss[2][kMaxStepTokens];       // sum of y^2 per column half

  // gate inputs of token gt (used by tid < 8); every load in the prologue is
  // unconditional, at a clamped index, so that none of them waits at a branch
  const int gh = r * g + jh, gt = tid & 7;  // gh = h
  const int64_t gi = ((int64_t)bseq * n + min(gt, n - 1)) * Hv + gh;
  const float ga = a[gi], gb = b[gi], gA = A_log[gh], gdt = dt_bias[gh];
  const __amdgpu_buffer_rsrc_t hrs = state_buf(state + ((int64_t)bseq * Hv + h) * kD * kD);
  const uint32_t hoff = (uint32_t)(d0 * kD + col) * (uint32_t)sizeof(float);
  f32x4 H[16];
  uint32_t zb[NT / 2], nwb;  // raw z bits of this lane's output tokens, norm weight bits

  // ---- prologue: conv + SiLU of every new token, 2 channels per thread ----------------
  // section = wave (waves 0-2): q, k, v.  raw[0..2] = cached rows (oldest first),
  // raw[3 + t] = new token t.  Only the v channels are advanced here (by their head's
  // workgroup); the q/k channels are advanced by qk_cache_advance_kernel afterwards.
  {
    T *cs = conv_state + (int64_t)bseq * 3 * Cc;
    const int c0 = lane * 2;
    // wave 3 repeats the q loads (channels no workgroup of this launch writes) and
    // stores nothing
    const int slot = wave == 3 ? 0 : wave;
    const bool active = wave < 3;
    const bool owner = wave == 2;   // v channels only
    int64_t cbase, hstride, sidx;
    const T *src;
    if (slot == 0) {
      cbase = (int64_t)g * kD; src = q; hstride = (int64_t)Hk * kD;
      sidx = ((int64_t)bseq * n * Hk + g) * kD;
    } else if (slot == 1) {
      cbase = (int64_t)Hk * kD + (int64_t)g * kD; src = k; hstride = (int64_t)Hk * kD;
      sidx = ((int64_t)bseq * n * Hk + g) * kD;
    } else {
      cbase = 2LL * Hk * kD + (int64_t)h * kD; src = v; hstride = (int64_t)Hv * kD;
      sidx = ((int64_t)bseq * n * Hv + h) * kD;
    }
    // the prologue's loads first, then the state's (one key row per register), so
    // that the state is in flight while the convolution waits for its inputs only
    // (raw bits; widened after the state loads have gone out)
    uint32_t rb[2][3 + NT];
    float4 w[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t ch = cbase + c0 + u;
      rb[u][0] = Act<T>::bits(cs, ch);
      rb[u][1] = Act<T>::bits(cs, Cc + ch);
      rb[u][2] = Act<T>::bits(cs, 2 * Cc + ch);
#pragma unroll
      for (int t = 0; t < NT; ++t)  // slots past n hold token n - 1 and are not used
        rb[u][3 + t] = Act<T>::bits(src, sidx + min(t, n - 1) * hstride + c0 + u);
      w[u] = *reinterpret_cast<const float4 *>(conv_w + ch * 4);
    }
    // the epilogue's inputs: z of the tokens this lane outputs (2 i + dh), the norm weight
#pragma unroll
    for (int i = 0; i < NT / 2; ++i)
      zb[i] = Act<T>::bits(z, (((int64_t)bseq * n + min(2 * i + dh, n - 1)) * Hv + h) * kD + col);
    nwb = norm_w ? __float_as_uint(norm_w[col]) : 0x3F800000u;
    __builtin_amdgcn_sched_barrier(0);  // keep the state loads behind these
#pragma unroll
    for (int m = 0; m < 16; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        H[m][i] = ld_row1(hrs, hoff, (4 * m + i) * kD * (int)sizeof(float));
    __builtin_amdgcn_sched_barrier(0);
    float raw[2][3 + NT];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 3 + NT; ++i) raw[u][i] = Act<T>::from_bits(rb[u][i]);
    float xv[NT][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t ch = cbase + c0 + u;
#pragma unroll
      for (int t = 0; t < NT; ++t)
        xv[t][u] = silu_fast(w[u].x * raw[u][t] + w[u].y * raw[u][t + 1] +
                             w[u].z * raw[u][t + 2] + w[u].w * raw[u][t + 3]);
      // the cache advances by `commit` tokens: rows commit .. commit + 2 of raw
      // (the reads above precede these writes, and only this thread touches ch)
      if (owner && commit > 0) {
#pragma unroll
        for (int s2 = 0; s2 < 3; ++s2) {
          float x = raw[u][0];
#pragma unroll
          for (int i = 1; i < 3 + NT; ++i)
            if (i == commit + s2) x = raw[u][i];
          Act<T>::store(cs, s2 * Cc + ch, x);
        }
      }
    }
    if (wave < 2) {  // L2-normalise q (wave 0) and k (wave 1) of each token
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t < n) {
          const float ss = wave_sum_dpp(xv[t][0] * xv[t][0] + xv[t][1] * xv[t][1]);
          const float f = (slot == 0 ? q_scale : 1.0f) * rsq_normal(ss + l2_eps);
          xv[t][0] *= f;
          xv[t][1] *= f;
        }
      }
    }
    if (active) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
        if (t < n) {
          s_x[t][slot][c0] = xv[t][0];
          s_x[t][slot][c0 + 1] = xv[t][1];
        }
    }
  }
  if (tid < 8 && gt < n) {
    s_ab[gt][0] = __expf(log_decay(ga, gA, gdt));
    s_ab[gt][1] = sigmoid_fast(gb);
  }
  __syncthreads();

  // ---- S_0 k_t and S_0 q_t over this wave's 64 key rows (MFMA) ------------------------
  // A operand of key rows d0 + 16 gq .. + 15: lane 4 b + i holds token 4 tg + i of row
  // d0 + 16 gq + b, so block abid = 4 mm + i of it pairs with register i of tile
  // 4 gq + mm.  Token slots past n read as zero.
  f32x4 Yk[NG], Yq[NG];
#pragma unroll
  for (int tg = 0; tg < NG; ++tg) Yk[tg] = Yq[tg] = f32x4{0.f, 0.f, 0.f, 0.f};
  {
    const int ti = lane & 3, di = lane >> 2;
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      float ak[NG], aq[NG];
#pragma unroll
      for (int tg = 0; tg < NG; ++tg) {
        const int t = 4 * tg + ti;
        const bool live = t < n;
        ak[tg] = live ? s_x[t][1][d0 + 16 * gq + di] : 0.f;
        aq[tg] = live ? s_x[t][0][d0 + 16 * gq + di] : 0.f;
      }
#pragma unroll
      for (int tg = 0; tg < NG; ++tg) {
        rows4<0>(ak[tg], aq[tg], H[4 * gq + 0], Yk[tg], Yq[tg]);
        rows4<4>(ak[tg], aq[tg], H[4 * gq + 1], Yk[tg], Yq[tg]);
        rows4<8>(ak[tg], aq[tg], H[4 * gq + 2], Yk[tg], Yq[tg]);
        rows4<12>(ak[tg], aq[tg], H[4 * gq + 3], Yk[tg], Yq[tg]);
      }
    }
  }
#pragma unroll
  for (int tg = 0; tg < NG; ++tg) {
    s_yp[dh][chh][2 * tg][lane] = Yk[tg];
    s_yp[dh][chh][2 * tg + 1][lane] = Yq[tg];
  }

  // ---- the n x n coefficients: token pairs s <= t dealt round-robin to the waves ------
  {
    int p = 0;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int s = 0; s <= t; ++s, ++p) {
        if (t < n && (p & 3) == wave) {
          const f32x2_t ks = *reinterpret_cast<const f32x2_t *>(&s_x[s][1][2 * lane]);
          const f32x2_t qt = *reinterpret_cast<const f32x2_t *>(&s_x[t][0][2 * lane]);
          const float kq = wave_sum_dpp(ks.x * qt.x + ks.y * qt.y);
          float kk = 0.f;
          if (s < t) {
            const f32x2_t kt = *reinterpret_cast<const f32x2_t *>(&s_x[t][1][2 * lane]);
            kk = wave_sum_dpp(ks.x * kt.x + ks.y * kt.y);
          }
          float R = 1.0f;
#pragma unroll
          for (int u = s + 1; u <= t; ++u) R *= s_ab[u][0];
          if (lane == 0) {
            s_cq[t][s] = R * kq;
            s_ck[t][s] = R * kk;
            s_R[t][s] = R;
            if (s == 0) s_G[t] = R * s_ab[0][0];
          }
        }
      }
    }
  }
  __syncthreads();

  // ---- per value column: the n x n recurrence for u_t and y_t -------------------------
#pragma unroll
  for (int tg = 0; tg < NG; ++tg) {
    Yk[tg] += s_yp[dh ^ 1][chh][2 * tg][lane];
    Yq[tg] += s_yp[dh ^ 1][chh][2 * tg + 1][lane];
  }
  float u[NT], y[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    u[t] = y[t] = 0.f;
    if (t < n) {
      const float Gt = s_G[t];
      float e = s_x[t][2][col] - Gt * Yk[t >> 2][t & 3];
#pragma unroll
      for (int s = 0; s < t; ++s) e -= s_ck[t][s] * u[s];
      u[t] = s_ab[t][1] * e;
      float yy = Gt * Yq[t >> 2][t & 3];
#pragma unroll
      for (int s = 0; s <= t; ++s) yy += s_cq[t][s] * u[s];
      y[t] = yy;
    }
  }

  // the two key-half waves of a column half hold the same y; the first one sums y^2
  if (dh == 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
      if (t < n) {
        const float ssum = wave_sum_dpp(y[t] * y[t]);
        if (lane == 0) s_ss[chh][t] = ssum;
      }
  }

  // ---- state after `commit` tokens: S_c = Gam_{c-1} S_0 + sum_s R_{c-1,s} u_s k_s^T ---
  // one MFMA per tile and token: A = k_s at key rows d0 + 4 m .. + 3 (block m of the
  // register holding k_s at row d0 + lane), B = R u_s at this lane's column.  Stored
  // before the epilogue's barrier, so that the stores are under way while it runs.
  if (commit > 0) {
    const float Gc = s_G[commit - 1];
#pragma unroll
    for (int m = 0; m < 16; ++m) H[m] *= Gc;
#pragma unroll
    for (int s = 0; s < NT; ++s) {
      if (s < commit) {
        const float w = s_R[commit - 1][s] * u[s];
        const float kd = s_x[s][1][d0 + lane];
        H[0] = outer4<0>(kd, w, H[0]);   H[1] = outer4<1>(kd, w, H[1]);
        H[2] = outer4<2>(kd, w, H[2]);   H[3] = outer4<3>(kd, w, H[3]);
        H[4] = outer4<4>(kd, w, H[4]);   H[5] = outer4<5>(kd, w, H[5]);
        H[6] = outer4<6>(kd, w, H[6]);   H[7] = outer4<7>(kd, w, H[7]);
        H[8] = outer4<8>(kd, w, H[8]);   H[9] = outer4<9>(kd, w, H[9]);
        H[10] = outer4<10>(kd, w, H[10]); H[11] = outer4<11>(kd, w, H[11]);
        H[12] = outer4<12>(kd, w, H[12]); H[13] = outer4<13>(kd, w, H[13]);
        H[14] = outer4<14>(kd, w, H[14]); H[15] = outer4<15>(kd, w, H[15]);
      }
    }
#pragma unroll
    for (int m = 0; m < 16; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        st_row1(hrs, hoff, (4 * m + i) * kD * (int)sizeof(float), H[m][i]);
  }

  // ---- epilogue: RMS over the head's 128 columns (two column halves), output gate -----
  // (z and the norm weight were loaded with the prologue); the key-half waves take
  // alternate tokens
  __syncthreads();
  {
    const float nwv = Act<float>::from_bits(nwb);
#pragma unroll
    for (int i = 0; i < NT / 2; ++i) {
      const int t = 2 * i + dh;
      if (t < n) {
        const int64_t oi = (((int64_t)bseq * n + t) * Hv + h) * kD + col;
        const float zr = Act<T>::from_bits(zb[i]);
        const float inv = rsq_normal((s_ss[0][t] + s_ss[1][t]) * (1.0f / kD) + rms_eps);
        const float sz = sigmoid_fast(zr);
        Act<T>::store(o, oi, y[t] * inv * nwv * (gate == 1 ? sz : zr * sz));
      }
    }
  }
}

// The q/k conv-cache channels advance by commit = num_commit[b] tokens after the
// n-token step has read them (same stream, so every read of the step precedes these
// writes): new row s = row commit + s of [cache rows, new tokens].  One thread per
// (sequence, V consecutive q/k channels), coalesced over channels; each thread reads
// its three source rows before it writes, and no other thread touches its channels.
template <typename T, int V>
__global__ void __launch_bounds__(256)
qk_cache_advance_kernel(const T *__restrict__ q, const T *__restrict__ k, T *__restrict__ conv_state,
                        const int32_t *__restrict__ num_commit, int batch, int Hk, int Hv, int n) {
  typedef T vec_t __attribute__((ext_vector_type(V)));
  const int64_t Cqk = 2LL * Hk * kD, groups = Cqk / V;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)batch * groups) return;
  const int bseq = (int)(i / groups);
  const int64_t ch = (i % groups) * V;
  const int commit = num_commit ? min(max(num_commit[bseq], 0), n) : n;
  if (commit == 0) return;
  const int64_t Cc = Cqk + (int64_t)Hv * kD;
  T *cs = conv_state + (int64_t)bseq * 3 * Cc + ch;
  const int64_t qkD = (int64_t)Hk * kD;
  const T *src = (ch < qkD ? q + ch : k + (ch - qkD)) + (int64_t)bseq * n * qkD;
  vec_t x[3];
#pragma unroll
  for (int s2 = 0; s2 < 3; ++s2) {
    const int j = commit + s2;  // 1 .. n + 2
    x[s2] = *reinterpret_cast<const vec_t *>(j < 3 ? cs + j * Cc : src + (j - 3) * qkD);
  }
#pragma unroll
  for (int s2 = 0; s2 < 3; ++s2) *reinterpret_cast<vec_t *>(cs + s2 * Cc) = x[s2];
}

template <typename T>
hipError_t launch_decode_tokens(const void *q, const void *k, const void *v, const float *a,
                                const float *b, const void *z, const float *conv_w,
                                const float *A_log, const float *dt_bias, const float *norm_w,
                                float q_scale, float l2_eps, float rms_eps, float *state,
                                void *conv_state, const int32_t *num_commit, void *o, int batch,
                                int n, int Hk, int Hv, int gate, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  dim3 grid((unsigned)batch * (unsigned)Hv);
  if (n <= 4)
    hipLaunchKernelGGL((decode_tokens_kernel<T, 1>), grid, dim3(kTokThreads), 0, stream,
                       (const T *)q, (const T *)k, (const T *)v, a, b, (const T *)z, conv_w,
                       A_log, dt_bias, norm_w, q_scale, l2_eps, rms_eps, state,
                       (T *)conv_state, num_commit, (T *)o, Hk, Hv, n, gate);
  else
    hipLaunchKernelGGL((decode_tokens_kernel<T, 2>), grid, dim3(kTokThreads), 0, stream,
                       (const T *)q, (const T *)k, (const T *)v, a, b, (const T *)z, conv_w,
                       A_log, dt_bias, norm_w, q_scale, l2_eps, rms_eps, state,
                       (T *)conv_state, num_commit, (T *)o, Hk, Hv, n, gate);
  // eight channels (one 16-byte access for bf16) per thread when the q, k and cache
  // pointers allow it, one channel otherwise
  const int64_t nch = (int64_t)batch * 2 * Hk * kD;
  const bool vec = (((uintptr_t)q | (uintptr_t)k | (uintptr_t)conv_state) % (8 * sizeof(T))) == 0;
  if (vec)
    hipLaunchKernelGGL((qk_cache_advance_kernel<T, 8>), dim3((unsigned)((nch / 8 + 255) / 256)),
                       dim3(256), 0, stream, (const T *)q, (const T *)k, (T *)conv_state,
                       num_commit, batch, Hk, Hv, n);
  else
    hipLaunchKernelGGL((qk_cache_advance_kernel<T, 1>), dim3((unsigned)((nch + 255) / 256)),
                       dim3(256), 0, stream, (const T *)q, (const T *)k, (T *)conv_state,
                       num_commit, batch, Hk, Hv, n);
  return hipGetLastError();
}

int decode_max_tokens() { return kMaxStepTokens; }

template hipError_t launch_decode_tokens<float>(const void *, const void *, const void *,
                                                const float *, const float *, const void *,
                                                const float *, const float *, const float *,
                                                const float *, float, float, float, float *,
                                                void *, const int32_t *, void *, int, int, int,
                                                int, int, hipStream_t);
template hipError_t launch_decode_tokens<bf16_t>(const void *, const void *, const void *,
                                                 const float *, const float *, const void *,
                                                 const float *, const float *, const float *,
                                                 const float *, float, float, float, float *,
                                                 void *, const int32_t *, void *, int, int, int,
                                                 int, int, hipStream_t);

}  // namespace gdn
