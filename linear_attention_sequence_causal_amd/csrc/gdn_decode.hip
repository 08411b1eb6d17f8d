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

template <typename T>
__global__ void __launch_bounds__(kDecThreads)
decode_step_kernel(const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
                   const float *__restrict__ a, const float *__restrict__ b,
                   const T *__restrict__ z, const float *__restrict__ conv_w,
                   const float *__restrict__ A_log, const float *__restrict__ dt_bias,
                   const float *__restrict__ norm_w, float q_scale, float l2_eps, float rms_eps,
                   float *__restrict__ state, T *__restrict__ conv_state, T *__restrict__ o,
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
  const float nwv = (norm_w && tid < kD) ? norm_w[tid] : 1.0f;
  float zcur = tid < kD ? Act<T>::load(z, ((int64_t)bseq * Hv + r * g) * kD + tid) : 0.f;
  // Start streaming the first head's state before the prologue.
  f32x4 Hcur[16];
  {
    const float *Hp = head_ptr(0);
#pragma unroll
    for (int i = 0; i < 16; ++i) Hcur[i] = ld_nt4(Hp + i * kD);
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
    const float zg = siluf_(zcur);
    if (j + 1 < r && tid < kD) zcur = Act<T>::load(z, ((int64_t)bseq * Hv + h + 1) * kD + tid);
    f32x4 Hnext[16];
    if (j + 1 < r) {
      const float *Hn = head_ptr(j + 1);
#pragma unroll
      for (int i = 0; i < 16; ++i) Hnext[i] = ld_nt4(Hn + i * kD);
    }
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
    float *Hp = head_ptr(j);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      f32x4 hn;
      hn.x = alpha * Hcur[i].x + kr[i] * ec[0];
      hn.y = alpha * Hcur[i].y + kr[i] * ec[1];
      hn.z = alpha * Hcur[i].z + kr[i] * ec[2];
      hn.w = alpha * Hcur[i].w + kr[i] * ec[3];
      st_nt4(Hp + i * kD, hn);
    }
    if (tid < kD) {
      const float inv = rsqrtf((s_misc[1] + s_misc[2]) * (1.0f / kD) + rms_eps);
      Act<T>::store(o, ((int64_t)bseq * Hv + h) * kD + tid, s_y[tid] * inv * nwv * zg);
    }
    __syncthreads();  // s_red, s_e, s_y, s_misc are reused by the next head
    if (j + 1 < r) {
#pragma unroll
      for (int i = 0; i < 16; ++i) Hcur[i] = Hnext[i];
    }
  }
}

template <typename T>
hipError_t launch_decode(const void *q, const void *k, const void *v, const float *a,
                         const float *b, const void *z, const float *conv_w, const float *A_log,
                         const float *dt_bias, const float *norm_w, float q_scale, float l2_eps,
                         float rms_eps, float *state, void *conv_state, void *o, int batch,
                         int Hk, int Hv, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  dim3 grid((unsigned)batch * (unsigned)Hk);
  hipLaunchKernelGGL((decode_step_kernel<T>), grid, dim3(kDecThreads), 0, stream,
                     (const T *)q, (const T *)k, (const T *)v, a, b, (const T *)z, conv_w, A_log,
                     dt_bias, norm_w, q_scale, l2_eps, rms_eps, state, (T *)conv_state, (T *)o,
                     Hk, Hv);
  return hipGetLastError();
}

int decode_max_ratio() { return kDecMaxRatio; }

template hipError_t launch_decode<float>(const void *, const void *, const void *, const float *,
                                         const float *, const void *, const float *,
                                         const float *, const float *, const float *, float,
                                         float, float, float *, void *, void *, int, int, int,
                                         hipStream_t);
template hipError_t launch_decode<bf16_t>(const void *, const void *, const void *,
                                          const float *, const float *, const void *,
                                          const float *, const float *, const float *,
                                          const float *, float, float, float, float *, void *,
                                          void *, int, int, int, hipStream_t);

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

template <typename T>
__global__ void __launch_bounds__(kDecThreads)
decode_tokens_kernel(const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
                     const float *__restrict__ a, const float *__restrict__ b,
                     const T *__restrict__ z, const float *__restrict__ conv_w,
                     const float *__restrict__ A_log, const float *__restrict__ dt_bias,
                     const float *__restrict__ norm_w, float q_scale, float l2_eps,
                     float rms_eps, float *__restrict__ state, T *__restrict__ conv_state,
                     const int32_t *__restrict__ num_commit, T *__restrict__ o, int Hk, int Hv,
                     int n) {
  const int g = blockIdx.x % Hk;
  const int bseq = blockIdx.x / Hk;
  const int r = Hv / Hk;
  const int tid = threadIdx.x;
  const int64_t Cc = 2LL * Hk * kD + (int64_t)Hv * kD;
  const int commit = num_commit ? min(max(num_commit[bseq], 0), n) : n;
  const float nwv = (norm_w && tid < kD) ? norm_w[tid] : 1.0f;  // loaded before the state

  __shared__ float s_x[kMaxStepTokens][2 + kDecMaxRatio][kD];  // post-prologue q, k, v rows
  __shared__ float s_red[8][2][kD];
  __shared__ float s_e[kD];
  __shared__ float s_y[kD];
  __shared__ float s_kq[kMaxStepTokens];
  __shared__ float s_ss[2];

  const int col = (tid & 31) * 4;
  const int rg = tid >> 5;
  const int row0 = rg * 16;
  auto head_ptr = [&](int j) {
    return state + (((int64_t)bseq * Hv + r * g + j) * kD + row0) * kD + col;
  };
  f32x4 Hcur[16];
  {
    const float *Hp = head_ptr(0);
#pragma unroll
    for (int i = 0; i < 16; ++i) Hcur[i] = ld_nt4(Hp + i * kD);
  }

  // ---- prologue: conv + SiLU of every new token, 2 channels per thread ----------------
  // raw[0..2] = cached rows (oldest first), raw[3 + t] = new token t
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
    const bool active = jv < r;
    int64_t cbase, hstride, sidx;
    const T *src;
    if (slot == 0) {
      cbase = (int64_t)g * kD; src = q; hstride = (int64_t)Hk * kD;
      sidx = ((int64_t)bseq * n * Hk + g) * kD;
    } else if (slot == 1) {
      cbase = (int64_t)Hk * kD + (int64_t)g * kD; src = k; hstride = (int64_t)Hk * kD;
      sidx = ((int64_t)bseq * n * Hk + g) * kD;
    } else {
      cbase = 2LL * Hk * kD + (int64_t)(r * g + jv) * kD; src = v; hstride = (int64_t)Hv * kD;
      sidx = ((int64_t)bseq * n * Hv + r * g + jv) * kD;
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
        // (reads above precede these writes; this thread owns the channel)
        if (commit > 0) {
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
    if (slot < 2) {  // L2-normalise q (wave 0) and k (wave 1) of each token over 128 channels
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
    if (active) {
#pragma unroll
      for (int t = 0; t < kMaxStepTokens; ++t)
        if (t < n) {
          s_x[t][slot][c0] = xv[t][0];
          s_x[t][slot][c0 + 1] = xv[t][1];
        }
    }
  }
  __syncthreads();
  if (tid < 64) {  // k_t . q_t of each token
    for (int t = 0; t < n; ++t) {
      const float kq = wave_sum(s_x[t][0][2 * tid] * s_x[t][1][2 * tid] +
                                s_x[t][0][2 * tid + 1] * s_x[t][1][2 * tid + 1]);
      if (tid == 0) s_kq[t] = kq;
    }
  }
  __syncthreads();

  // ---- per v head: the state stays in registers across the n tokens ------------------
  // Gate inputs and z of every token of a head are loaded before its token loop, so
  // no global load latency sits between two tokens.
  float ga[kMaxStepTokens], gb[kMaxStepTokens], zr[kMaxStepTokens];
  auto load_head_inputs = [&](int h) {
#pragma unroll
    for (int t = 0; t < kMaxStepTokens; ++t) {
      const int64_t gi = ((int64_t)bseq * n + min(t, n - 1)) * Hv + h;
      ga[t] = a[gi];
      gb[t] = b[gi];
      zr[t] = tid < kD ? Act<T>::load(z, gi * kD + tid) : 0.f;
    }
  };
  load_head_inputs(r * g);
  for (int j = 0; j < r; ++j) {
    const int h = r * g + j;
    float alph[kMaxStepTokens], bet[kMaxStepTokens], zg[kMaxStepTokens];
#pragma unroll
    for (int t = 0; t < kMaxStepTokens; ++t) {
      alph[t] = __expf(log_decay(ga[t], A_log[h], dt_bias[h]));
      bet[t] = sigmoidf_(gb[t]);
      zg[t] = siluf_(zr[t]);
    }
    // the next head's small inputs, then its state: vector-memory waits are in
    // issue order, so nothing waited on in the token loop queues behind the state
    if (j + 1 < r) load_head_inputs(h + 1);
    f32x4 Hnext[16];
    if (j + 1 < r) {
      const float *Hn = head_ptr(j + 1);
#pragma unroll
      for (int i = 0; i < 16; ++i) Hnext[i] = ld_nt4(Hn + i * kD);
    }
#pragma unroll
    for (int t = 0; t < kMaxStepTokens; ++t) {
      if (t >= n) break;
      const int64_t gi = ((int64_t)bseq * n + t) * Hv + h;
      const float alpha = alph[t];
      const float beta = bet[t];
      float kr[16], qr[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        kr[i] = s_x[t][1][row0 + i];
        qr[i] = s_x[t][0][row0 + i];
      }
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
        const float e = s_x[t][2 + j][tid] - alpha * vk;  // e = v - S'k
        const float y = alpha * vq + beta * s_kq[t] * e;  // S'' q
        s_e[tid] = e;
        s_y[tid] = y;
        const float ssum = wave_sum(y * y);
        if ((tid & 63) == 0) s_ss[tid >> 6] = ssum;
      }
      __syncthreads();
      float ec[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) ec[c] = beta * s_e[col + c];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        Hcur[i].x = alpha * Hcur[i].x + kr[i] * ec[0];
        Hcur[i].y = alpha * Hcur[i].y + kr[i] * ec[1];
        Hcur[i].z = alpha * Hcur[i].z + kr[i] * ec[2];
        Hcur[i].w = alpha * Hcur[i].w + kr[i] * ec[3];
      }
      if (t + 1 == commit) {
        float *Hp = head_ptr(j);
#pragma unroll
        for (int i = 0; i < 16; ++i) st_nt4(Hp + i * kD, Hcur[i]);
      }
      if (tid < kD) {
        const float inv = rsqrtf((s_ss[0] + s_ss[1]) * (1.0f / kD) + rms_eps);
        Act<T>::store(o, gi * kD + tid, s_y[tid] * inv * nwv * zg[t]);
      }
    }
    __syncthreads();  // s_red, s_e, s_y, s_ss are reused by the next head
    if (j + 1 < r) {
#pragma unroll
      for (int i = 0; i < 16; ++i) Hcur[i] = Hnext[i];
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
  dim3 grid((unsigned)batch * (unsigned)Hk);
  hipLaunchKernelGGL((decode_tokens_kernel<T>), grid, dim3(kDecThreads), 0, stream,
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
