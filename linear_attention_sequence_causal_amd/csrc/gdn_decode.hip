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
constexpr int kDecMaxRatio = 8;  // largest Hv / Hk the decode kernel accepts

// Stored state: fp32, or bf16 (rounded to nearest even on every store) with the
// step itself computed in fp32.  Four consecutive columns per access, streamed
// once (non-temporal).  A prefetched head is kept in its stored form (Raw) until
// it is used, so bf16 storage needs half the registers for it.
template <typename S> struct StateIO;
template <> struct StateIO<float> {
  typedef f32x4 Raw;
  static __device__ __forceinline__ Raw load_raw(const float *p) { return ld_nt4(p); }
  static __device__ __forceinline__ f32x4 widen(Raw x) { return x; }
  static __device__ __forceinline__ f32x4 load(const float *p) { return ld_nt4(p); }
  static __device__ __forceinline__ void store(float *p, f32x4 x) { st_nt4(p, x); }
};
template <> struct StateIO<bf16_t> {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  typedef u32x2 Raw;
  static __device__ __forceinline__ Raw load_raw(const bf16_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
  }
  static __device__ __forceinline__ f32x4 widen(Raw w) {
    return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                 __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u)};
  }
  static __device__ __forceinline__ f32x4 load(const bf16_t *p) { return widen(load_raw(p)); }
  static __device__ __forceinline__ void store(bf16_t *p, f32x4 x) {
    const u32x2 w = {pk_bf16(x.x, x.y), pk_bf16(x.z, x.w)};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2 *>(p));
  }
};

template <typename T, typename S>
__global__ void __launch_bounds__(kDecThreads)
decode_step_kernel(const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
                   const float *__restrict__ a, const float *__restrict__ b,
                   const T *__restrict__ z, const float *__restrict__ conv_w,
                   const float *__restrict__ A_log, const float *__restrict__ dt_bias,
                   const float *__restrict__ norm_w, float q_scale, float l2_eps, float rms_eps,
                   S *__restrict__ state, T *__restrict__ conv_state, T *__restrict__ o,
                   int Hk, int Hv) {
  const int g = blockIdx.x % Hk;
  const int bseq = blockIdx.x / Hk;
  const int r = Hv / Hk;
  const int tid = threadIdx.x;
  const int64_t Cc = 2LL * Hk * kD + (int64_t)Hv * kD;

  __shared__ float s_x[2 + kDecMaxRatio][kD];  // post-prologue q, k, then v of each v head
  __shared__ float s_red[8][2][kD];            // partial column sums per row group
  __shared__ float s_e[kD];
  __shared__ float s_y[kD];
  __shared__ float s_misc[4];

  // thread t of the state stream: columns 4*(t%32)..+3, rows 16*(t/32)..+15
  const int col = (tid & 31) * 4;
  const int rg = tid >> 5;
  const int row0 = rg * 16;
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
  typename StateIO<S>::Raw Hraw[16];
  {
    const S *Hp = head_ptr(0);
#pragma unroll
    for (int i = 0; i < 16; ++i) Hraw[i] = StateIO<S>::load_raw(Hp + i * kD);
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
        xv[u] = siluf_(w.x * h0 + w.y * h1 + w.z * h2 + w.w * raw);
        // shift the cache in place (reads above precede these writes)
        Act<T>::store(cs, ch, h1);
        Act<T>::store(cs, Cc + ch, h2);
        Act<T>::store(cs, 2 * Cc + ch, raw);
      }
    }
    if (slot < 2) {  // L2-normalise q (wave 0) and k (wave 1) over 128 channels
      const float ss = wave_sum(xv[0] * xv[0] + xv[1] * xv[1]);
      const float f = (slot == 0 ? q_scale : 1.0f) * rsqrtf(ss + l2_eps);
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
    const float kq = wave_sum(s_x[0][2 * tid] * s_x[1][2 * tid] +
                              s_x[0][2 * tid + 1] * s_x[1][2 * tid + 1]);
    if (tid == 0) s_misc[0] = kq;
  }
  __syncthreads();
  const float kq = s_misc[0];

  float kr[16], qr[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    kr[i] = s_x[1][row0 + i];
    qr[i] = s_x[0][row0 + i];
  }

  // ---- 3./4. per v head: state stream and epilogue ---------------------------------
  for (int j = 0; j < r; ++j) {
    const int h = r * g + j;
    const float zg = siluf_(Act<T>::from_bits(zbits));
    if (j + 1 < r) zbits = Act<T>::bits(z, ((int64_t)bseq * Hv + h + 1) * kD + ztid);
    // the next head's loads go out first (vector-memory waits are in issue order, so
    // waiting for this head's state does not wait for them)
    typename StateIO<S>::Raw Hnext[16];
    if (j + 1 < r) {
      const S *Hn = head_ptr(j + 1);
#pragma unroll
      for (int i = 0; i < 16; ++i) Hnext[i] = StateIO<S>::load_raw(Hn + i * kD);
    }
    f32x4 Hcur[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) Hcur[i] = StateIO<S>::widen(Hraw[i]);
    const float alpha = __expf(log_decay(a[(int64_t)bseq * Hv + h], A_log[h], dt_bias[h]));
    const float beta = sigmoidf_(b[(int64_t)bseq * Hv + h]);
    float sk[4] = {0, 0, 0, 0}, sq[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sk[0] += Hcur[i].x * kr[i]; sk[1] += Hcur[i].y * kr[i];
      sk[2] += Hcur[i].z * kr[i]; sk[3] += Hcur[i].w * kr[i];
      sq[0] += Hcur[i].x * qr[i]; sq[1] += Hcur[i].y * qr[i];
      sq[2] += Hcur[i].z * qr[i]; sq[3] += Hcur[i].w * qr[i];
    }
    *reinterpret_cast<f32x4 *>(&s_red[rg][0][col]) = f32x4{sk[0], sk[1], sk[2], sk[3]};
    *reinterpret_cast<f32x4 *>(&s_red[rg][1][col]) = f32x4{sq[0], sq[1], sq[2], sq[3]};
    __syncthreads();
    if (tid < kD) {
      float vk = 0.f, vq = 0.f;
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        vk += s_red[p][0][tid];
        vq += s_red[p][1][tid];
      }
      const float e = s_x[2 + j][tid] - alpha * vk;  // e = v - S'k
      const float y = alpha * vq + beta * kq * e;    // S'' q
      s_e[tid] = e;
      s_y[tid] = y;
      const float ssum = wave_sum(y * y);
      if ((tid & 63) == 0) s_misc[1 + (tid >> 6)] = ssum;
    }
    __syncthreads();
    float ec[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) ec[c] = beta * s_e[col + c];
    S *Hp = head_ptr(j);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      f32x4 hn;
      hn.x = alpha * Hcur[i].x + kr[i] * ec[0];
      hn.y = alpha * Hcur[i].y + kr[i] * ec[1];
      hn.z = alpha * Hcur[i].z + kr[i] * ec[2];
      hn.w = alpha * Hcur[i].w + kr[i] * ec[3];
      StateIO<S>::store(Hp + i * kD, hn);
    }
    if (tid < kD) {
      const float inv = rsqrtf((s_misc[1] + s_misc[2]) * (1.0f / kD) + rms_eps);
      Act<T>::store(o, ((int64_t)bseq * Hv + h) * kD + tid, s_y[tid] * inv * nwv * zg);
    }
    __syncthreads();  // s_red, s_e, s_y, s_misc are reused by the next head
    if (j + 1 < r) {
#pragma unroll
      for (int i = 0; i < 16; ++i) Hraw[i] = Hnext[i];
    }
  }
}

// state_bf16: the state is bf16 storage (void * either way)
template <typename T>
hipError_t launch_decode(const void *q, const void *k, const void *v, const float *a,
                         const float *b, const void *z, const float *conv_w, const float *A_log,
                         const float *dt_bias, const float *norm_w, float q_scale, float l2_eps,
                         float rms_eps, void *state, bool state_bf16, void *conv_state, void *o,
                         int batch, int Hk, int Hv, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  dim3 grid((unsigned)batch * (unsigned)Hk);
  if (state_bf16)
    hipLaunchKernelGGL((decode_step_kernel<T, bf16_t>), grid, dim3(kDecThreads), 0, stream,
                       (const T *)q, (const T *)k, (const T *)v, a, b, (const T *)z, conv_w,
                       A_log, dt_bias, norm_w, q_scale, l2_eps, rms_eps, (bf16_t *)state,
                       (T *)conv_state, (T *)o, Hk, Hv);
  else
    hipLaunchKernelGGL((decode_step_kernel<T, float>), grid, dim3(kDecThreads), 0, stream,
                       (const T *)q, (const T *)k, (const T *)v, a, b, (const T *)z, conv_w,
                       A_log, dt_bias, norm_w, q_scale, l2_eps, rms_eps, (float *)state,
                       (T *)conv_state, (T *)o, Hk, Hv);
  return hipGetLastError();
}

int decode_max_ratio() { return kDecMaxRatio; }

template hipError_t launch_decode<float>(const void *, const void *, const void *, const float *,
                                         const float *, const void *, const float *,
                                         const float *, const float *, const float *, float,
                                         float, float, void *, bool, void *, void *, int, int,
                                         int, hipStream_t);
template hipError_t launch_decode<bf16_t>(const void *, const void *, const void *,
                                          const float *, const float *, const void *,
                                          const float *, const float *, const float *,
                                          const float *, float, float, float, void *, bool,
                                          void *, void *, int, int, int, hipStream_t);

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

// One workgroup of four waves per (sequence, v head): wave w holds value columns
// 32 w + 2 cg, + 1 (cg = lane & 15) and key rows 32 rg .. + 31 (rg = lane >> 4) of the
// fp32 state, 64 values per lane, so that four waves fit on a SIMD and the state
// reads of some workgroups overlap the token loops of others.  The r workgroups of a
// q/k head each convolve its q and k rows (the first of them advances their conv
// cache).  A token's S k and S q sums are finished across the four row lanes with
// permlane swaps, so the token loop needs no LDS round trip and no barrier; the RMS
// of each token's y (split over the four waves) is taken once after the loop.
constexpr int kTokThreads = 256;
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
// One v head's fp32 state as a raw buffer: each lane's 8-byte pieces are addressed by
// its own offset plus a uniform row offset, so no per-row 64-bit addresses are kept
// in registers.  Cache policy non-temporal (the state is touched once per call).
constexpr int kNtPolicy = 2;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t state_buf(float *base) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, kD * kD * (int)sizeof(float),
                                           0x00020000);
}
__device__ __forceinline__ f32x2_t ld_row2(__amdgpu_buffer_rsrc_t r, uint32_t off, int row_off) {
  return __builtin_bit_cast(f32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, row_off, kNtPolicy));
}
__device__ __forceinline__ void st_row2(__amdgpu_buffer_rsrc_t r, uint32_t off, int row_off,
                                        f32x2_t x) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, x), r, off, row_off,
                                        kNtPolicy);
}

template <typename T>
__global__ void __launch_bounds__(kTokThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
decode_tokens_kernel(const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
                     const float *__restrict__ a, const float *__restrict__ b,
                     const T *__restrict__ z, const float *__restrict__ conv_w,
                     const float *__restrict__ A_log, const float *__restrict__ dt_bias,
                     const float *__restrict__ norm_w, float q_scale, float l2_eps,
                     float rms_eps, float *__restrict__ state, T *__restrict__ conv_state,
                     const int32_t *__restrict__ num_commit, T *__restrict__ o, int Hk, int Hv,
                     int n) {
  const int r = Hv / Hk;
  const int jh = blockIdx.x % r;                  // v head within its q/k group
  const int g = (blockIdx.x / r) % Hk;            // q/k head
  const int bseq = blockIdx.x / r / Hk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t Cc = 2LL * Hk * kD + (int64_t)Hv * kD;
  const int commit = num_commit ? min(max(num_commit[bseq], 0), n) : n;

  // v head (the clamp is a no-op; in this form the kernel fits 128 registers unspilled)
  const int h = r * g + min(jh, r - 1);
  const int cg = lane & 15, rg = lane >> 4;
  const int col0 = 32 * (wave & 3) + 2 * cg;      // 2 value columns
  const int row0 = 32 * rg;                       // 32 key rows
  const int ocol = col0 + (rg & 1);               // the column this lane outputs
  const bool out_lane = rg < 2;                   // rows 2, 3 repeat rows 0, 1

  __shared__ float s_x[kMaxStepTokens][3][kD];    // post-prologue q, k, v rows
  __shared__ float s_kq[kMaxStepTokens];
  __shared__ float s_ss[4][kMaxStepTokens];       // per-wave partial sums of y^2
  __shared__ float s_ab[kMaxStepTokens][2];       // alpha, beta of each token
  __shared__ float s_y[4][kMaxStepTokens][64];    // y of each lane's output column

  // the gate inputs first; the state is read after the prologue, whose registers it
  // would otherwise share (four waves per SIMD need at most 128 registers per lane)
  float ga = 0.f, gb = 0.f;  // gate inputs of token gt (tid < 8)
  const int gh = r * g + jh, gt = tid & 7;  // gh = h
  if (tid < 8 && gt < n) {
    const int64_t gi = ((int64_t)bseq * n + gt) * Hv + gh;
    ga = a[gi];
    gb = b[gi];
  }
  const __amdgpu_buffer_rsrc_t hrs = state_buf(state + ((int64_t)bseq * Hv + h) * kD * kD);
  const uint32_t hoff = (uint32_t)(row0 * kD + col0) * (uint32_t)sizeof(float);
  f32x2_t Hs[32];

  // ---- prologue: conv + SiLU of every new token, 2 channels per thread ----------------
  // section = wave (waves 0-2): q, k, v.  raw[0..2] = cached rows (oldest first),
  // raw[3 + t] = new token t.  The q/k cache channels belong to the workgroup of the
  // group's first v head, the v channels to their head's workgroup.
  {
    T *cs = conv_state + (int64_t)bseq * 3 * Cc;
    const int c0 = lane * 2;
    const int slot = wave;
    const bool active = slot < 3;
    const bool owner = slot < 2 ? jh == 0 : true;
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
    float xv[kMaxStepTokens][2];
#pragma unroll
    for (int t = 0; t < kMaxStepTokens; ++t) xv[t][0] = xv[t][1] = 0.f;
    if (active) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int64_t ch = cbase + c0 + u;
        float raw[3 + kMaxStepTokens];
        raw[0] = Act<T>::load(cs, ch);
        raw[1] = Act<T>::load(cs, Cc + ch);
        raw[2] = Act<T>::load(cs, 2 * Cc + ch);
#pragma unroll
        for (int t = 0; t < kMaxStepTokens; ++t)
          raw[3 + t] = t < n ? Act<T>::load(src, sidx + t * hstride + c0 + u) : 0.f;
        const float4 w = *reinterpret_cast<const float4 *>(conv_w + ch * 4);
#pragma unroll
        for (int t = 0; t < kMaxStepTokens; ++t)
          xv[t][u] = siluf_(w.x * raw[t] + w.y * raw[t + 1] + w.z * raw[t + 2] + w.w * raw[t + 3]);
        // the cache advances by `commit` tokens: rows commit .. commit + 2 of raw
        // (the reads above precede these writes, and only this thread touches ch)
        if (owner && commit > 0) {
#pragma unroll
          for (int s2 = 0; s2 < 3; ++s2) {
            float x = raw[0];
#pragma unroll
            for (int i = 1; i < 3 + kMaxStepTokens; ++i)
              if (i == commit + s2) x = raw[i];
            Act<T>::store(cs, s2 * Cc + ch, x);
          }
        }
      }
    }
    if (slot < 2) {  // L2-normalise q (wave 0) and k (wave 1) of each token
#pragma unroll
      for (int t = 0; t < kMaxStepTokens; ++t) {
        if (t < n) {
          const float ss = wave_sum(xv[t][0] * xv[t][0] + xv[t][1] * xv[t][1]);
          const float f = (slot == 0 ? q_scale : 1.0f) * rsqrtf(ss + l2_eps);
          xv[t][0] *= f;
          xv[t][1] *= f;
        }
      }
    }
    if (slot < 3) {
#pragma unroll
      for (int t = 0; t < kMaxStepTokens; ++t)
        if (t < n) {
          s_x[t][slot][c0] = xv[t][0];
          s_x[t][slot][c0 + 1] = xv[t][1];
        }
    }
  }
  // the state (the barriers below do not wait for these loads)
#pragma unroll
  for (int i = 0; i < 32; ++i) Hs[i] = ld_row2(hrs, hoff, i * kD * (int)sizeof(float));
  if (tid < 8 && gt < n) {
    s_ab[gt][0] = __expf(log_decay(ga, A_log[gh], dt_bias[gh]));
    s_ab[gt][1] = sigmoidf_(gb);
  }
  __syncthreads();
  if (wave == 0) {  // k_t . q_t of each token
    for (int t = 0; t < n; ++t) {
      const float kq = wave_sum(s_x[t][0][2 * lane] * s_x[t][1][2 * lane] +
                                s_x[t][0][2 * lane + 1] * s_x[t][1][2 * lane + 1]);
      if (lane == 0) s_kq[t] = kq;
    }
  }
  __syncthreads();

  // ---- token loop: the state stays in registers, no barrier -----------------------------
  // The registers hold the state divided by the running decay product of this call,
  // S = Gam * Hs, so a token costs one FMA per state element for the update instead
  // of a decay multiply and an FMA: with Gam_t = alpha_t Gam_{t-1},
  //   alpha_t S_{t-1} k = Gam_t (Hs k),  S_t = Gam_t (Hs + (beta e / Gam_t) k^T).
  // When Gam_t falls below 2^-60 it is folded into Hs (and taken as 1), which also
  // covers alpha = 0.  Gam is uniform (one head per workgroup).
  float Gam = 1.0f;
#pragma unroll 1
  for (int t = 0; t < n; ++t) {
    {
      const float alpha = s_ab[t][0];
      const float beta = s_ab[t][1];
      float Gt = Gam * alpha;
      if (Gt < 0x1p-60f) {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          Hs[i].x *= Gt; Hs[i].y *= Gt;
        }
        Gt = 1.0f;
      }
      Gam = Gt;
      // k and q rows 32 rg .. + 31 are read from LDS in blocks of 4 (broadcast
      // within each 16-lane row); k again for the update, to keep registers low
      float sk[2] = {0, 0}, sq[2] = {0, 0};
#pragma unroll
      for (int i = 0; i < 32; i += 4) {
        const f32x4 kk = *reinterpret_cast<const f32x4 *>(&s_x[t][1][row0 + i]);
        const f32x4 qq = *reinterpret_cast<const f32x4 *>(&s_x[t][0][row0 + i]);
        const float kv[4] = {kk.x, kk.y, kk.z, kk.w}, qv[4] = {qq.x, qq.y, qq.z, qq.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const f32x2_t hv = Hs[i + u];
          sk[0] += hv.x * kv[u]; sk[1] += hv.y * kv[u];
          sq[0] += hv.x * qv[u]; sq[1] += hv.y * qv[u];
        }
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        sk[c] = rows4_sum(sk[c]);
        sq[c] = rows4_sum(sq[c]);
      }
      const f32x2_t vv = *reinterpret_cast<const f32x2_t *>(&s_x[t][2][col0]);
      const float kq = s_kq[t];
      float be[2];
      float y[2];
      const float vs[2] = {vv.x, vv.y};
      const float rG = 1.0f / Gt;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const float e = vs[c] - Gt * sk[c];   // e = v - S'k
        y[c] = Gt * sq[c] + beta * kq * e;    // S_t q
        be[c] = beta * e * rG;
      }
      s_y[wave][t][lane] = (rg & 1) ? y[1] : y[0];
#pragma unroll
      for (int i = 0; i < 32; i += 4) {
        const f32x4 kk = *reinterpret_cast<const f32x4 *>(&s_x[t][1][row0 + i]);
        const float kv[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          Hs[i + u].x = fmaf(kv[u], be[0], Hs[i + u].x);
          Hs[i + u].y = fmaf(kv[u], be[1], Hs[i + u].y);
        }
      }
      if (t + 1 == commit) {
#pragma unroll
        for (int i = 0; i < 32; ++i)
          st_row2(hrs, hoff, i * kD * (int)sizeof(float), f32x2_t{Gam * Hs[i].x, Gam * Hs[i].y});
      }
    }
  }

  // ---- epilogue: RMS over the head's 128 columns (four waves), SiLU(z) gate -----------
  const float nwv = norm_w ? norm_w[ocol] : 1.0f;
  float zr[kMaxStepTokens];
#pragma unroll
  for (int t = 0; t < kMaxStepTokens; ++t)
    zr[t] = Act<T>::load(z, (((int64_t)bseq * n + min(t, n - 1)) * Hv + h) * kD + ocol);
  float yown[kMaxStepTokens];
#pragma unroll
  for (int t = 0; t < kMaxStepTokens; ++t) {
    yown[t] = t < n ? s_y[wave][t][lane] : 0.f;  // this lane's own writes: no barrier
    if (t < n) {
      // each column sits in one of the lanes with rg < 2: sum over those
      const float ssum = wave_sum(out_lane ? yown[t] * yown[t] : 0.f);
      if (lane == 0) s_ss[wave][t] = ssum;
    }
  }
  __syncthreads();
  if (out_lane) {
#pragma unroll
    for (int t = 0; t < kMaxStepTokens; ++t) {
      if (t < n) {
        const float ssh = (s_ss[0][t] + s_ss[1][t]) + (s_ss[2][t] + s_ss[3][t]);
        const float inv = rsqrtf(ssh * (1.0f / kD) + rms_eps);
        const int64_t oi = (((int64_t)bseq * n + t) * Hv + h) * kD + ocol;
        Act<T>::store(o, oi, yown[t] * inv * nwv * siluf_(zr[t]));
      }
    }
  }
}

template <typename T>
hipError_t launch_decode_tokens(const void *q, const void *k, const void *v, const float *a,
                                const float *b, const void *z, const float *conv_w,
                                const float *A_log, const float *dt_bias, const float *norm_w,
                                float q_scale, float l2_eps, float rms_eps, float *state,
                                void *conv_state, const int32_t *num_commit, void *o, int batch,
                                int n, int Hk, int Hv, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  dim3 grid((unsigned)batch * (unsigned)Hv);
  hipLaunchKernelGGL((decode_tokens_kernel<T>), grid, dim3(kTokThreads), 0, stream,
                     (const T *)q, (const T *)k, (const T *)v, a, b, (const T *)z, conv_w, A_log,
                     dt_bias, norm_w, q_scale, l2_eps, rms_eps, state, (T *)conv_state,
                     num_commit, (T *)o, Hk, Hv, n);
  return hipGetLastError();
}

int decode_max_tokens() { return kMaxStepTokens; }

template hipError_t launch_decode_tokens<float>(const void *, const void *, const void *,
                                                const float *, const float *, const void *,
                                                const float *, const float *, const float *,
                                                const float *, float, float, float, float *,
                                                void *, const int32_t *, void *, int, int, int,
                                                int, hipStream_t);
template hipError_t launch_decode_tokens<bf16_t>(const void *, const void *, const void *,
                                                 const float *, const float *, const void *,
                                                 const float *, const float *, const float *,
                                                 const float *, float, float, float, float *,
                                                 void *, const int32_t *, void *, int, int, int,
                                                 int, hipStream_t);

}  // namespace gdn
