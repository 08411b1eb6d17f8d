// gdn_prefill.hip -- chunked prefill of the Gated DeltaNet mixer on gfx950.
//
// Method (rows = tokens of one 64-token chunk, H = S^T [dk][dv] the state the
// chunk enters with, g = log alpha, G = chunk-local cumsum of g, gamma = e^G):
//   L[i][j] = beta_i e^{G_i-G_j} (k_i . k_j)  (j < i)      T = (I + L)^-1
//   W       = T diag(beta gamma) K                         Utilde = T diag(beta) V
//   U       = Utilde - W H                                 ("v_new")
//   M[i][j] = e^{G_i-G_j} (q_i . k_j)  (j <= i)
//   O       = diag(gamma) Q H + M U                        (y of every token)
//   H      <- gamma_C H + K^T diag(e^{G_C-G}) U            (state * chunk_decay + key^T v_new)
// This is the six update steps of the "Qwen3-Next 80B-A3B" field guide
// (cutaway 02) unrolled over a chunk; its state line is the chunk update of the
// "Qwen3.8-Flash-Next" model card.  The prologue (width-4 causal conv + SiLU,
// L2 norm of q and k, gates g = -exp(A_log) softplus(a + dt_bias),
// beta = sigmoid(b)) and the gated RMSNorm epilogue are fused into the chunk
// loop, so q/k/v/z/a/b are read once and o is written once.
//
// Precision plan (bf16 MFMA operands, fp32 accumulation, fp32 state):
//   Q K^T and the state update K^T U use split operands x = hi + lo
//   (hi*hi + hi*lo + lo*hi); K K^T, W, T V, W H, Q H and M U use one bf16
//   pass; the identity part of T V (beta V) and the diagonal of M U are
//   applied in fp32.  The triangular inverse is exact in fp32 on its 16x16
//   diagonal blocks and merged with bf16 products.
//
// Work decomposition: one workgroup = 8 waves = one (segment, v head); wave w
// owns value columns 16w..16w+15 of the state in MFMA accumulators.  Long
// sequences are cut into segments: pass 1 computes each non-final segment's
// affine map H -> A H + B (the same chunk loop run on the columns of A = I and
// B = 0), pass 2 chains the maps into segment start states, pass 3 runs the
// full chunk loop of every segment from its start state.
#include "gdn_device.h"
#include "gdn_prefill_plan.h"

namespace gdn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(u16x8 a, u16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ u16x8 cat4(u16x4 x, u16x4 y) {
  return u16x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
}

// --------------------------------------------------------------------- LDS
constexpr int kThreads = 512;  // 8 waves
constexpr int kWaves = 8;
constexpr int kRowS = 136;     // bf16 row stride of [64 tok][128 d] tiles (272 B)
constexpr int kTokS = 72;      // bf16 row stride of [128 d][64 tok] tiles (144 B)
constexpr int kSqS = 68;       // row stride of [64][64] tiles (fp32 L/T, bf16 M/X)

constexpr int OFF_QH = 0;
constexpr int OFF_QL = OFF_QH + 64 * kRowS * 2;
constexpr int OFF_KH = OFF_QL + 64 * kRowS * 2;
constexpr int OFF_KL = OFF_KH + 64 * kRowS * 2;
constexpr int OFF_KTH = OFF_KL + 64 * kRowS * 2;
constexpr int OFF_KTL = OFF_KTH + 128 * kTokS * 2;
constexpr int OFF_VTH = OFF_KTL + 128 * kTokS * 2;
constexpr int OFF_VTL = OFF_VTH + 128 * kTokS * 2;
constexpr int OFF_CONVW = OFF_VTL + 128 * kTokS * 2;
constexpr int OFF_BETA = OFF_CONVW + 384 * 4 * 4;
constexpr int OFF_G = OFF_BETA + 64 * 4;
constexpr int OFF_MDIAG = OFF_G + 64 * 4;
constexpr int OFF_RMS = OFF_MDIAG + 64 * 4;
constexpr int kLdsBytes = OFF_RMS + kWaves * 64 * 4;
// reused regions after the gram products
constexpr int OFF_L = OFF_KH;              // fp32 [64][68], then T in place
constexpr int OFF_M = OFF_KL;              // bf16 [64][68]  M with zero diagonal
constexpr int OFF_XW = OFF_QL;             // bf16 [64][68]  T diag(beta gamma)
constexpr int OFF_XU = OFF_QL + 64 * kSqS * 2;  // bf16 [64][68]  (T - I) diag(beta)
constexpr int OFF_W = OFF_KH;              // bf16 [64][136] -W (after T is consumed)
static_assert(OFF_XU + 64 * kSqS * 2 <= OFF_KH, "X tiles overflow the Q-lo region");
static_assert(64 * kSqS * 4 <= 64 * kRowS * 2, "L does not fit the K-hi region");
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");

enum Mode { kFull = 0, kMapA = 1, kMapB = 2 };

struct PrefillArgs {
  const void *q, *k, *v, *z;
  const float *a, *b;
  const float *conv_w, *A_log, *dt_bias, *norm_w;
  float q_scale, l2_eps, rms_eps;
  const float *init_state;
  const void *conv_in;
  void *o;
  float *final_state;
  const SegInfo *segs;
  const int32_t *hdr;      // [0] segments, [1] maps
  const int32_t *map_seg;  // map slot -> segment index
  float *maps;             // [max_maps][Hv][2][D][D]
  float *starts;           // [max_segments][Hv][D][D]
  int Hk, Hv;
  int64_t Cc;
  int precise_all;         // split-precision state update on every chunk
};

template <typename T> struct Raw;  // 8 channels of one token as raw 32-bit words
template <> struct Raw<bf16_t> {
  static constexpr int W = 4;  // words per 8 channels
  static __device__ __forceinline__ void load(uint32_t (&dst)[W], const bf16_t *p) {
    const uint4 t = *reinterpret_cast<const uint4 *>(p);
    dst[0] = t.x; dst[1] = t.y; dst[2] = t.z; dst[3] = t.w;
  }
  static __device__ __forceinline__ float get(const uint32_t (&w)[W], int c) {
    const uint32_t word = w[c >> 1];
    return __uint_as_float((c & 1) ? (word & 0xFFFF0000u) : (word << 16));
  }
};
template <> struct Raw<float> {
  static constexpr int W = 8;
  static __device__ __forceinline__ void load(uint32_t (&dst)[W], const float *p) {
    const uint4 t0 = *reinterpret_cast<const uint4 *>(p);
    const uint4 t1 = *reinterpret_cast<const uint4 *>(p + 4);
    dst[0] = t0.x; dst[1] = t0.y; dst[2] = t0.z; dst[3] = t0.w;
    dst[4] = t1.x; dst[5] = t1.y; dst[6] = t1.z; dst[7] = t1.w;
  }
  static __device__ __forceinline__ float get(const uint32_t (&w)[W], int c) {
    return __uint_as_float(w[c]);
  }
};

__device__ __forceinline__ uint32_t pack2(bf16_t lo, bf16_t hi) {
  return (uint32_t)lo | ((uint32_t)hi << 16);
}

// hi/lo bf16 split of 8 floats, packed as two 16-byte words
__device__ __forceinline__ void split_pack8(const float (&x)[8], uint4 &hi, uint4 &lo) {
  bf16_t h[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) split_bf(x[i], h[i], l[i]);
  hi = make_uint4(pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7]));
  lo = make_uint4(pack2(l[0], l[1]), pack2(l[2], l[3]), pack2(l[4], l[5]), pack2(l[6], l[7]));
}

// Width-4 causal conv + SiLU of NT tokens x 8 channels.  raw[r] holds the raw
// inputs of token tbase - 3 + r of the chunk; wv the 8 x 4 taps (tap 3 = current
// token).  Tokens at or past nvalid (the padded tail of a partial chunk) are 0.
template <typename T, int NT>
__device__ __forceinline__ void conv_silu_rows(const uint32_t (&raw)[11][Raw<T>::W],
                                               const float *wv, int tbase, int nvalid,
                                               float (&x)[NT][8]) {
  float w[8][4];
#pragma unroll
  for (int cc = 0; cc < 8; ++cc) {
    const f32x4 t = *reinterpret_cast<const f32x4 *>(wv + cc * 4);
    w[cc][0] = t.x; w[cc][1] = t.y; w[cc][2] = t.z; w[cc][3] = t.w;
  }
#pragma unroll
  for (int r = 0; r < NT; ++r) {
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) acc += w[cc][j] * Raw<T>::get(raw[r + j], cc);
      x[r][cc] = (tbase + r < nvalid) ? siluf_(acc) : 0.f;
    }
  }
}

// ------------------------------------------------------------ chunk kernel
template <typename T, int MODE>
__global__ void __launch_bounds__(kThreads, 1) chunk_kernel(PrefillArgs P) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int tid = threadIdx.x;
  int wave = tid >> 6, lane = tid & 63;
  int ln = lane & 15, lg = lane >> 4;  // MFMA lane coordinates
  const int Hv = P.Hv, Hk = P.Hk;
  const int h = blockIdx.x % Hv;
  const int unit = blockIdx.x / Hv;  // segment (full) or map slot (map modes)
  const int gq = h / (Hv / Hk);

  int segi;
  if (MODE == kFull) {
    if (unit >= P.hdr[0]) return;
    segi = unit;
  } else {
    if (unit >= P.hdr[1]) return;
    segi = P.map_seg[unit];
  }
  const SegInfo seg = P.segs[segi];
  const int seq_begin = seg.seq_begin;
  const int seg_end = seg.begin + seg.len;

  bf16_t *const sQh = reinterpret_cast<bf16_t *>(smem + OFF_QH);
  bf16_t *const sQl = reinterpret_cast<bf16_t *>(smem + OFF_QL);
  bf16_t *const sKh = reinterpret_cast<bf16_t *>(smem + OFF_KH);
  bf16_t *const sKl = reinterpret_cast<bf16_t *>(smem + OFF_KL);
  bf16_t *const sKTh = reinterpret_cast<bf16_t *>(smem + OFF_KTH);
  bf16_t *const sKTl = reinterpret_cast<bf16_t *>(smem + OFF_KTL);
  bf16_t *const sVTh = reinterpret_cast<bf16_t *>(smem + OFF_VTH);
  bf16_t *const sVTl = reinterpret_cast<bf16_t *>(smem + OFF_VTL);
  float *const sConvW = reinterpret_cast<float *>(smem + OFF_CONVW);
  float *const sBeta = reinterpret_cast<float *>(smem + OFF_BETA);
  float *const sG = reinterpret_cast<float *>(smem + OFF_G);
  float *const sMdiag = reinterpret_cast<float *>(smem + OFF_MDIAG);
  float *const sRms = reinterpret_cast<float *>(smem + OFF_RMS);
  float *const sL = reinterpret_cast<float *>(smem + OFF_L);
  bf16_t *const sM = reinterpret_cast<bf16_t *>(smem + OFF_M);
  bf16_t *const sXw = reinterpret_cast<bf16_t *>(smem + OFF_XW);
  bf16_t *const sXu = reinterpret_cast<bf16_t *>(smem + OFF_XU);
  bf16_t *const sW = reinterpret_cast<bf16_t *>(smem + OFF_W);

  // ---- roles of the prologue ----------------------------------------------------
  // threads 0..127: q, 128..255: k (8 channels x 8 tokens each),
  // 256..511: v (8 channels x 4 tokens each).  Map mode A needs no q, v.
  const int role = tid < 128 ? 0 : (tid < 256 ? 1 : 2);
  const int ridx = role == 2 ? tid - 256 : (tid & 127);
  int cg = ridx & 15;                      // channels 8cg .. 8cg+7
  const int tg = ridx >> 4;                // token group
  const int NT = role == 2 ? 4 : 8;        // tokens per thread
  int tbase = tg * NT;
  // Re-derive the lane coordinates behind an optimisation barrier after every
  // workgroup barrier, so that LDS addresses are formed next to their use
  // instead of being hoisted out of the chunk loop (and spilled).
  auto refresh = [&]() {
    tid = opaque(tid);
    wave = tid >> 6;
    lane = tid & 63;
    ln = lane & 15;
    lg = lane >> 4;
    cg = opaque(cg);
    tbase = opaque(tbase);
  };
  int64_t cbase;  // conv channel of this thread's first channel
  if (role == 0) cbase = (int64_t)gq * kD;
  else if (role == 1) cbase = (int64_t)Hk * kD + (int64_t)gq * kD;
  else cbase = 2LL * Hk * kD + (int64_t)h * kD;
  const bool role_on = MODE == kFull || (role == 1) || (MODE == kMapB && role == 2);

  // conv weights of this head's 384 channels -> LDS (q 0..127, k 128..255, v 256..383)
  for (int i = tid; i < 384 * 4; i += kThreads) {
    const int ch = i >> 2, tap = i & 3;
    int64_t c;
    if (ch < 128) c = (int64_t)gq * kD + ch;
    else if (ch < 256) c = (int64_t)Hk * kD + (int64_t)gq * kD + (ch - 128);
    else c = 2LL * Hk * kD + (int64_t)h * kD + (ch - 256);
    sConvW[i] = P.conv_w[c * 4 + tap];
  }

  const T *src = role == 0 ? (const T *)P.q : (role == 1 ? (const T *)P.k : (const T *)P.v);
  const int64_t tok_stride = role == 2 ? (int64_t)Hv * kD : (int64_t)Hk * kD;
  const int64_t head_off = (role == 2 ? (int64_t)h : (int64_t)gq) * kD + cg * 8;
  const T *hist = P.conv_in ? (const T *)P.conv_in + (int64_t)seg.seq * 3 * P.Cc + cbase + cg * 8
                            : nullptr;

  // raw rows for one chunk: rows tbase-3 .. tbase+NT-1 relative to the chunk start
  constexpr int RW = Raw<T>::W;
  uint32_t raw[11][RW];
  float ga = 0.f, gb = 0.f;  // gate inputs of token `lane` (wave 7)
  auto load_chunk = [&](int t0) {
    if (role_on) {
#pragma unroll
      for (int rr = 0; rr < 11; ++rr) {
        if (rr < NT + 3) {
          const int tau = t0 + tbase - 3 + rr;
          if (tau >= seq_begin && tau < seg_end) {
            Raw<T>::load(raw[rr], src + (int64_t)tau * tok_stride + head_off);
          } else if (tau < seq_begin && hist) {
            Raw<T>::load(raw[rr], hist + (int64_t)(3 + tau - seq_begin) * P.Cc);
          } else {
#pragma unroll
            for (int w = 0; w < RW; ++w) raw[rr][w] = 0u;
          }
        }
      }
    }
    if (wave == 7) {
      const int tau = t0 + lane;
      if (tau < seg_end) {
        ga = P.a[(int64_t)tau * Hv + h];
        gb = P.b[(int64_t)tau * Hv + h];
      }
    }
  };

  // ---- state accumulators ---------------------------------------------------------
  // Hacc[dt]: rows (dk) 16dt + 4lg + i, column (dv) 16*wave + ln.
  f32x4 Hacc[8];
  {
    const float *H0 = nullptr;
    if (MODE == kFull) {
      if (seg.nseg > 1) H0 = P.starts + ((int64_t)segi * Hv + h) * kD * kD;
      else if (P.init_state) H0 = P.init_state + ((int64_t)seg.seq * Hv + h) * kD * kD;
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * dt + 4 * lg + i, col = 16 * wave + ln;
        float x = 0.f;
        if (MODE == kFull) x = H0 ? H0[row * kD + col] : 0.f;
        else if (MODE == kMapA) x = row == col ? 1.f : 0.f;
        Hacc[dt][i] = x;
      }
  }

  const float A_log_h = P.A_log[h], dt_bias_h = P.dt_bias[h];
  const int nchunks = (seg.len + kChunk - 1) / kChunk;
  const bool last_seg = seg.idx == seg.nseg - 1;
  if (nchunks > 0) load_chunk(seg.begin);
  __syncthreads();  // conv weights

  for (int c = 0; c < nchunks; ++c) {
    refresh();
    const int t0 = seg.begin + c * kChunk;
    const int nvalid = min(kChunk, seg_end - t0);

    // ================= prologue: conv + SiLU (+ L2), gates -> LDS ================
    if (role_on) {
      const float *wv = sConvW + ((role * 128) + cg * 8) * 4;
      if (role < 2) {  // q or k: 8 tokens x 8 channels, L2 over the head's 128 channels
        float x[8][8];
        conv_silu_rows<T, 8>(raw, wv, tbase, nvalid, x);
        const float scale0 = role == 0 ? P.q_scale : 1.0f;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          float ss = 0.f;
#pragma unroll
          for (int cc = 0; cc < 8; ++cc) ss += x[r][cc] * x[r][cc];
          ss = group_sum<16>(ss);
          const float f = scale0 * rsqrtf(ss + P.l2_eps);
#pragma unroll
          for (int cc = 0; cc < 8; ++cc) x[r][cc] *= f;
        }
        bf16_t *dh = role == 0 ? sQh : sKh;
        bf16_t *dl = role == 0 ? sQl : sKl;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          uint4 hi, lo;
          split_pack8(x[r], hi, lo);
          const int off = (tbase + r) * kRowS + cg * 8;
          *reinterpret_cast<uint4 *>(dh + off) = hi;
          *reinterpret_cast<uint4 *>(dl + off) = lo;
        }
        if (role == 1) {  // K^T [dk][tok], 8 tokens per channel = 16 bytes
#pragma unroll
          for (int cc = 0; cc < 8; ++cc) {
            float col[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) col[r] = x[r][cc];
            uint4 hi, lo;
            split_pack8(col, hi, lo);
            const int off = (cg * 8 + cc) * kTokS + tbase;
            *reinterpret_cast<uint4 *>(sKTh + off) = hi;
            *reinterpret_cast<uint4 *>(sKTl + off) = lo;
          }
        }
      } else {  // v: 4 tokens x 8 channels -> V^T [dv][tok], 8 bytes per channel
        float x[4][8];
        conv_silu_rows<T, 4>(raw, wv, tbase, nvalid, x);
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) {
          bf16_t hi[4], lo[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) split_bf(x[r][cc], hi[r], lo[r]);
          const int off = (cg * 8 + cc) * kTokS + tbase;
          *reinterpret_cast<uint2 *>(sVTh + off) = make_uint2(pack2(hi[0], hi[1]), pack2(hi[2], hi[3]));
          *reinterpret_cast<uint2 *>(sVTl + off) = make_uint2(pack2(lo[0], lo[1]), pack2(lo[2], lo[3]));
        }
      }
    }
    if (wave == 7) {  // gates of token `lane`, inclusive cumsum of g
      float g = 0.f, be = 0.f;
      if (lane < nvalid) {
        g = log_decay(ga, A_log_h, dt_bias_h);
        be = sigmoidf_(gb);
      }
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float up = __shfl_up(g, o, 64);
        if (lane >= o) g += up;
      }
      sBeta[lane] = be;
      sG[lane] = g;
    }
    __syncthreads();  // (1) prologue tiles ready
    refresh();

    // prefetch the next chunk's raw rows (consumed by the next prologue)
    if (c + 1 < nchunks) load_chunk(t0 + kChunk);

    // ================= gram products K K^T (and Q K^T) =========================
    // lower tiles (i, j), j <= i: wave w takes tile w, waves 0 and 1 also 8, 9
    f32x4 kk[2], qk[2];
    const int ntiles = wave < 2 ? 2 : 1;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      kk[s] = f32x4{0, 0, 0, 0};
      qk[s] = f32x4{0, 0, 0, 0};
      if (s < ntiles) {
        const int t = wave + 8 * s;
        const int ti = (t >= 1) + (t >= 3) + (t >= 6);  // lower tiles in row order
        const int tj = t - ti * (ti + 1) / 2;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const int col = 32 * kb + 8 * lg;
          const u16x8 bk = *reinterpret_cast<const u16x8 *>(sKh + (16 * tj + ln) * kRowS + col);
          const u16x8 ak = *reinterpret_cast<const u16x8 *>(sKh + (16 * ti + ln) * kRowS + col);
          kk[s] = mfma16(ak, bk, kk[s]);
          if (MODE == kFull) {
            const u16x8 bkl = *reinterpret_cast<const u16x8 *>(sKl + (16 * tj + ln) * kRowS + col);
            const u16x8 aqh = *reinterpret_cast<const u16x8 *>(sQh + (16 * ti + ln) * kRowS + col);
            const u16x8 aql = *reinterpret_cast<const u16x8 *>(sQl + (16 * ti + ln) * kRowS + col);
            qk[s] = mfma16(aqh, bk, qk[s]);
            qk[s] = mfma16(aqh, bkl, qk[s]);
            qk[s] = mfma16(aql, bk, qk[s]);
          }
        }
      }
    }
    __syncthreads();  // (2) K tiles consumed: L and M overwrite them
    refresh();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (s < ntiles) {
        const int t = wave + 8 * s;
        const int ti = (t >= 1) + (t >= 3) + (t >= 6);
        const int tj = t - ti * (ti + 1) / 2;
        const int cj = 16 * tj + ln;
        const float Gj = sG[cj];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ri = 16 * ti + 4 * lg + i;
          const float Gi = sG[ri];
          const bool low = cj < ri;
          const float d = __expf(low ? Gi - Gj : 0.f);
          sL[ri * kSqS + cj] = low ? sBeta[ri] * d * kk[s][i] : 0.f;
          if (MODE == kFull) {
            sM[ri * kSqS + cj] = f2bf(low ? d * qk[s][i] : 0.f);
            if (cj == ri) sMdiag[ri] = qk[s][i];
          }
        }
      }
    }
    if (MODE == kFull && wave < 2) {  // zero upper tiles (0,1) and (2,3) of M read by M U
      const int ti = wave == 0 ? 0 : 2;
#pragma unroll
      for (int i = 0; i < 4; ++i) sM[(16 * ti + 4 * lg + i) * kSqS + 16 * (ti + 1) + ln] = 0;
    }
    __syncthreads();  // (3) L, M ready
    refresh();

    // ================= triangular inverse (wave 0) | Q H, beta V (all) ============
    if (wave == 0) {
      // (a) 16x16 diagonal blocks by forward substitution; lane = (block, column)
      {
        const int bb = lg, cc = ln;
        float *Lb = sL + (16 * bb) * kSqS + 16 * bb;
        float xcol[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float sacc = (r == cc) ? 1.f : 0.f;
#pragma unroll
          for (int j = 0; j < r; ++j) sacc -= Lb[r * kSqS + j] * xcol[j];
          xcol[r] = sacc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) Lb[r * kSqS + cc] = xcol[r];
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      // (b) 16 -> 32: T[b1][b0] = -T[b1][b1] (L[b1][b0] T[b0][b0]) for (0,1) and (2,3)
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const int b0 = 2 * pr, b1 = 2 * pr + 1;
        u16x8 A, B;
#pragma unroll
        for (int j = 0; j < 8; ++j) {  // natural k order, K = 16 real of 32
          const int kx = 8 * lg + j;
          A[j] = kx < 16 ? f2bf(sL[(16 * b1 + ln) * kSqS + 16 * b0 + kx]) : 0;
          B[j] = kx < 16 ? f2bf(sL[(16 * b0 + kx) * kSqS + 16 * b0 + ln]) : 0;
        }
        f32x4 Pm = mfma16(A, B, f32x4{0, 0, 0, 0});  // P = L10 T00
#pragma unroll
        for (int j = 0; j < 8; ++j) {  // k slot 8lg + j <-> k = 4lg + j (j < 4)
          A[j] = j < 4 ? f2bf(sL[(16 * b1 + ln) * kSqS + 16 * b1 + 4 * lg + j]) : 0;
          B[j] = j < 4 ? f2bf(Pm[j]) : 0;
        }
        f32x4 Tm = mfma16(A, B, f32x4{0, 0, 0, 0});
#pragma unroll
        for (int i = 0; i < 4; ++i) sL[(16 * b1 + 4 * lg + i) * kSqS + 16 * b0 + ln] = -Tm[i];
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      // (c) 32 -> 64: T[23][01] = -T[23][23] (L[23][01] T[01][01])
      {
        f32x4 P2[2][2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int nj = 0; nj < 2; ++nj) {
            u16x8 A, B;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int kx = 8 * lg + j;  // 0..31, natural
              A[j] = f2bf(sL[(32 + 16 * mi + ln) * kSqS + kx]);
              const bool zero = (nj == 1 && kx < 16);  // upper block T01 = 0
              B[j] = zero ? 0 : f2bf(sL[kx * kSqS + 16 * nj + ln]);
            }
            P2[mi][nj] = mfma16(A, B, f32x4{0, 0, 0, 0});
          }
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int nj = 0; nj < 2; ++nj) {
            u16x8 A, B;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              // k slot 8lg + j <-> k = 4lg + j (j < 4) or 16 + 4lg + (j - 4)
              const int kx = j < 4 ? 4 * lg + j : 16 + 4 * lg + (j - 4);
              const bool zero = (mi == 0 && kx >= 16);  // upper block T23 = 0
              A[j] = zero ? 0 : f2bf(sL[(32 + 16 * mi + ln) * kSqS + 32 + kx]);
              B[j] = f2bf(j < 4 ? P2[0][nj][j] : P2[1][nj][j - 4]);
            }
            f32x4 Tm = mfma16(A, B, f32x4{0, 0, 0, 0});
#pragma unroll
            for (int i = 0; i < 4; ++i)
              sL[(32 + 16 * mi + 4 * lg + i) * kSqS + 16 * nj + ln] = -Tm[i];
          }
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      // (d) X_w = T diag(beta gamma), X_u = (T - I) diag(beta); lane = column
      {
        const int cc = lane;
        const float bcol = sBeta[cc];
        const float bgcol = bcol * __expf(sG[cc]);
#pragma unroll 8
        for (int r = 0; r < 64; ++r) {
          const float t = (cc <= r) ? sL[r * kSqS + cc] : 0.f;
          sXw[r * kSqS + cc] = f2bf(t * bgcol);
          sXu[r * kSqS + cc] = f2bf(cc < r ? t * bcol : 0.f);
        }
      }
    }

    // H as bf16 B operands: Hb[kb] slots 8lg+j <-> dk 32kb + 4lg + j (j<4), 32kb+16+4lg+j-4
    u16x8 Hb[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        Hb[kb][j] = f2bf(Hacc[2 * kb][j]);
        Hb[kb][4 + j] = f2bf(Hacc[2 * kb + 1][j]);
      }
    f32x4 Oacc[4], Uacc[4];
    int dvc = 16 * wave + ln;  // this lane's value column
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      Oacc[mt] = f32x4{0, 0, 0, 0};
      Uacc[mt] = f32x4{0, 0, 0, 0};
      if (MODE == kFull) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const bf16_t *qrow = sQh + (16 * mt + ln) * kRowS + 32 * kb + 4 * lg;
          const u16x8 aq = cat4(*reinterpret_cast<const u16x4 *>(qrow),
                                *reinterpret_cast<const u16x4 *>(qrow + 16));
          Oacc[mt] = mfma16(aq, Hb[kb], Oacc[mt]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) Oacc[mt][i] *= __expf(sG[16 * mt + 4 * lg + i]);
      }
      if (MODE != kMapA) {  // identity part of Utilde: beta V, from V^T hi + lo
        const int toff = dvc * kTokS + 16 * mt + 4 * lg;
        const u16x4 vh = *reinterpret_cast<const u16x4 *>(sVTh + toff);
        const u16x4 vl = *reinterpret_cast<const u16x4 *>(sVTl + toff);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          Uacc[mt][i] = sBeta[16 * mt + 4 * lg + i] * (bf2f(vh[i]) + bf2f(vl[i]));
      }
    }
    __syncthreads();  // (4) T, X_w, X_u ready; L consumed
    refresh();
    dvc = 16 * wave + ln;

    // ================= W = T diag(beta gamma) K (dk tile = wave); Utilde += X_u V ====
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 wacc = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb == 1 && mt < 2) continue;  // T is lower triangular
        const bf16_t *xr = sXw + (16 * mt + ln) * kSqS + 32 * kb + 8 * lg;
        const u16x8 ax = cat4(*reinterpret_cast<const u16x4 *>(xr),
                              *reinterpret_cast<const u16x4 *>(xr + 4));
        const u16x8 bk = *reinterpret_cast<const u16x8 *>(sKTh + dvc * kTokS + 32 * kb + 8 * lg);
        wacc = mfma16(ax, bk, wacc);
        if (MODE != kMapA) {
          const bf16_t *ur = sXu + (16 * mt + ln) * kSqS + 32 * kb + 8 * lg;
          const u16x8 au = cat4(*reinterpret_cast<const u16x4 *>(ur),
                                *reinterpret_cast<const u16x4 *>(ur + 4));
          const u16x8 bv = *reinterpret_cast<const u16x8 *>(sVTh + dvc * kTokS + 32 * kb + 8 * lg);
          Uacc[mt] = mfma16(au, bv, Uacc[mt]);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sW[(16 * mt + 4 * lg + i) * kRowS + dvc] = f2bf(-wacc[i]);
    }
    __syncthreads();  // (5) -W ready
    refresh();
    dvc = 16 * wave + ln;

    // ================= chain: U = Utilde - W H; O += M U; H update ===============
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const bf16_t *wr = sW + (16 * mt + ln) * kRowS + 32 * kb + 4 * lg;
        const u16x8 aw = cat4(*reinterpret_cast<const u16x4 *>(wr),
                              *reinterpret_cast<const u16x4 *>(wr + 16));
        Uacc[mt] = mfma16(aw, Hb[kb], Uacc[mt]);
      }
    // U as B operands (k = token): Ub[kb] slots <-> tokens 32kb + 4lg + j, 32kb+16+4lg+j-4
    if (MODE == kFull) {
      u16x8 Ub[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          Ub[kb][j] = f2bf(Uacc[2 * kb][j]);
          Ub[kb][4 + j] = f2bf(Uacc[2 * kb + 1][j]);
        }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if (kb == 1 && mt < 2) continue;
          const bf16_t *mr = sM + (16 * mt + ln) * kSqS + 32 * kb + 4 * lg;
          const u16x8 am = cat4(*reinterpret_cast<const u16x4 *>(mr),
                                *reinterpret_cast<const u16x4 *>(mr + 16));
          Oacc[mt] = mfma16(am, Ub[kb], Oacc[mt]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) Oacc[mt][i] += sMdiag[16 * mt + 4 * lg + i] * Uacc[mt][i];
      }
    }
    // state update H = gamma_C H + K^T diag(e^{G_C - G}) U
    {
      const float GC = sG[63];
      const float gC = __expf(GC);
      u16x8 Uh[2], Ul[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int mt = 2 * kb + (j >> 2);
          const int tok = 16 * mt + 4 * lg + (j & 3);
          const float u = Uacc[mt][j & 3] * __expf(GC - sG[tok]);
          bf16_t hi, lo;
          split_bf(u, hi, lo);
          Uh[kb][j] = hi;
          Ul[kb][j] = lo;
        }
      // the final state gets the split-precision update over its last two chunks
      const bool precise = MODE == kFull && (P.precise_all || (last_seg && c >= nchunks - 2));
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) Hacc[dt][i] *= gC;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int off = (16 * dt + ln) * kTokS + 32 * kb + 4 * lg;
          const u16x8 akh = cat4(*reinterpret_cast<const u16x4 *>(sKTh + off),
                                 *reinterpret_cast<const u16x4 *>(sKTh + off + 16));
          Hacc[dt] = mfma16(akh, Uh[kb], Hacc[dt]);
          if (precise) {
            const u16x8 akl = cat4(*reinterpret_cast<const u16x4 *>(sKTl + off),
                                   *reinterpret_cast<const u16x4 *>(sKTl + off + 16));
            Hacc[dt] = mfma16(akh, Ul[kb], Hacc[dt]);
            Hacc[dt] = mfma16(akl, Uh[kb], Hacc[dt]);
          }
        }
      }
    }

    // ================= epilogue: RMSNorm over 128 columns, SiLU(z) gate ============
    if (MODE == kFull) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float s = group_sum<16>(Oacc[mt][i] * Oacc[mt][i]);
          if (ln == 0) sRms[wave * 64 + 16 * mt + 4 * lg + i] = s;
        }
    }
    __syncthreads();  // (6) partial sums ready; all LDS tiles of this chunk consumed
    refresh();
    dvc = 16 * wave + ln;
    if (MODE == kFull) {
      const float wn = P.norm_w ? P.norm_w[dvc] : 1.0f;
      T *op = (T *)P.o;
      const T *zp = (const T *)P.z;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = 16 * mt + 4 * lg + i;
          if (tok < nvalid) {
            float ss = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) ss += sRms[w * 64 + tok];
            const float inv = rsqrtf(ss * (1.0f / kD) + P.rms_eps);
            const int64_t idx = ((int64_t)(t0 + tok) * Hv + h) * kD + dvc;
            const float zv = Act<T>::load(zp, idx);
            Act<T>::store(op, idx, Oacc[mt][i] * inv * wn * siluf_(zv));
          }
        }
    }
  }

  // ---- state out ---------------------------------------------------------------------
  float *Hout = nullptr;
  if (MODE == kFull) {
    if (last_seg) Hout = P.final_state + ((int64_t)seg.seq * Hv + h) * kD * kD;
  } else {
    Hout = P.maps + (((int64_t)unit * Hv + h) * 2 + (MODE == kMapA ? 0 : 1)) * kD * kD;
  }
  if (Hout) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) Hout[(16 * dt + 4 * lg + i) * kD + 16 * wave + ln] = Hacc[dt][i];
  }
}

// ------------------------------------------------------------ segment table
// One workgroup: sequence lengths -> segments (prefix sums over sequences).
__global__ void __launch_bounds__(1024) segment_table_kernel(
    const int32_t *cu, int N, int64_t T, int seg_len, int64_t max_segments, int64_t max_maps,
    SegInfo *segs, int32_t *hdr, int32_t *map_seg) {
  __shared__ int s_nseg[1024], s_nmap[1024];
  __shared__ int s_base_seg, s_base_map;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_base_seg = 0;
    s_base_map = 0;
  }
  __syncthreads();
  for (int n0 = 0; n0 < N; n0 += 1024) {
    const int n = n0 + tid;
    int b = 0, e = 0, ns = 0, nm = 0, nch = 0;
    if (n < N) {
      b = cu ? cu[n] : 0;
      e = cu ? cu[n + 1] : (int)T;
      b = max(0, min(b, (int)T));       // keep every access inside [0, T)
      e = max(b, min(e, (int)T));
      const int len = e - b;
      ns = len == 0 ? 1 : (len + seg_len - 1) / seg_len;
      nm = ns - 1;
      nch = (len + kChunk - 1) / kChunk;
    }
    s_nseg[tid] = ns;
    s_nmap[tid] = nm;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {  // inclusive scans
      const int a1 = tid >= o ? s_nseg[tid - o] : 0;
      const int a2 = tid >= o ? s_nmap[tid - o] : 0;
      __syncthreads();
      s_nseg[tid] += a1;
      s_nmap[tid] += a2;
      __syncthreads();
    }
    const int first = s_base_seg + s_nseg[tid] - ns;
    const int firstmap = s_base_map + s_nmap[tid] - nm;
    if (n < N) {
      // chunks are spread evenly over the segments (the first nch % ns get one
      // more), so every segment of a split sequence holds >= 4 full chunks
      const int q = nch / ns, rem = nch % ns;
      for (int s = 0; s < ns; ++s) {
        const int idx = first + s;
        if (idx >= max_segments) break;
        SegInfo si;
        si.seq = n;
        si.begin = b + kChunk * (s * q + min(s, rem));
        si.len = max(0, min(kChunk * (q + (s < rem ? 1 : 0)), e - si.begin));
        si.idx = s;
        si.nseg = ns;
        si.first = first;
        si.map = (s < ns - 1 && firstmap + s < max_maps) ? firstmap + s : -1;
        si.seq_begin = b;
        segs[idx] = si;
        if (si.map >= 0) map_seg[si.map] = idx;
      }
    }
    __syncthreads();
    if (tid == 1023) {
      s_base_seg += s_nseg[1023];
      s_base_map += s_nmap[1023];
    }
    __syncthreads();
  }
  if (tid == 0) {
    // More segments than the bound means cu_seqlens was invalid (overlapping or
    // not ending at T): run nothing rather than index past the tables.
    const bool ok = s_base_seg <= max_segments && s_base_map <= max_maps;
    hdr[0] = ok ? s_base_seg : 0;
    hdr[1] = ok ? s_base_map : 0;
  }
}

// ------------------------------------------------------------ combine (pass 2)
// Per (sequence, v head, 16-column slice): H_0 = init; H_{s+1} = A_s H_s + B_s,
// written as the start state of every segment of a multi-segment sequence.
__global__ void __launch_bounds__(256) combine_kernel(const SegInfo *segs, const int32_t *hdr,
                                                      const float *init_state, const float *maps,
                                                      float *starts, int Hv) {
  __shared__ float sH[kD][17];
  const int slice = blockIdx.x % 8;
  const int h = (blockIdx.x / 8) % Hv;
  const int segi = blockIdx.x / (8 * Hv);  // candidate first segment
  if (segi >= hdr[0]) return;
  const SegInfo s0 = segs[segi];
  if (s0.idx != 0 || s0.nseg < 2) return;
  const int tid = threadIdx.x;
  const int row = tid >> 1, c0 = (tid & 1) * 8;  // 8 outputs per thread
  const int col0 = slice * 16 + c0;
  float hreg[8];
  const float *H0 = init_state ? init_state + ((int64_t)s0.seq * Hv + h) * kD * kD : nullptr;
#pragma unroll
  for (int j = 0; j < 8; ++j) hreg[j] = H0 ? H0[row * kD + col0 + j] : 0.f;
  for (int s = 0; s < s0.nseg; ++s) {
    float *dst = starts + ((int64_t)(segi + s) * Hv + h) * kD * kD;
#pragma unroll
    for (int j = 0; j < 8; ++j) dst[row * kD + col0 + j] = hreg[j];
    if (s == s0.nseg - 1) break;
    const int m = segs[segi + s].map;
    const float *A = maps + (((int64_t)m * Hv + h) * 2 + 0) * kD * kD;
    const float *B = maps + (((int64_t)m * Hv + h) * 2 + 1) * kD * kD;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) sH[row][c0 + j] = hreg[j];
    __syncthreads();
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = B[row * kD + col0 + j];
    for (int kx = 0; kx < kD; ++kx) {
      const float a = A[row * kD + kx];
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] += a * sH[kx][c0 + j];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) hreg[j] = acc[j];
  }
}

// ------------------------------------------------------------ conv state out
// Last three raw inputs of every sequence (inherited history when shorter).
template <typename T>
__global__ void conv_out_kernel(const int32_t *cu, int N, int64_t T_total, const T *q, const T *k,
                                const T *v, const T *conv_in, T *conv_out, int Hk, int Hv,
                                int64_t Cc) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)N * Cc) return;
  const int n = (int)(i / Cc);
  const int64_t c = i % Cc;
  int b = cu ? cu[n] : 0, e = cu ? cu[n + 1] : (int)T_total;
  b = max(0, min(b, (int)T_total));
  e = max(b, min(e, (int)T_total));
  const int len = e - b;
  T vals[3];
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    const int tau = len - 3 + r;
    if (tau >= 0) {
      const int64_t t = b + tau;
      if (c < (int64_t)Hk * kD) vals[r] = q[t * Hk * kD + c];
      else if (c < 2LL * Hk * kD) vals[r] = k[t * Hk * kD + (c - (int64_t)Hk * kD)];
      else vals[r] = v[t * Hv * kD + (c - 2LL * Hk * kD)];
    } else {
      vals[r] = conv_in ? conv_in[((int64_t)n * 3 + 3 + tau) * Cc + c] : (T)0;
    }
  }
#pragma unroll
  for (int r = 0; r < 3; ++r) conv_out[((int64_t)n * 3 + r) * Cc + c] = vals[r];
}

// ------------------------------------------------------------ host side
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Segment length: the smallest power of two >= 512 (at most 8192 tokens)
// that still gives about one workgroup per compute unit over all v heads.
static int32_t pick_seg_len(int64_t T, int32_t Hv) {
  int64_t target = T * (int64_t)Hv / 256;
  int32_t s = 512;
  while (s < 8192 && s < target) s *= 2;
  return s;
}

PrefillPlan make_plan(int32_t num_seqs, int64_t total_tokens, int32_t num_v_heads) {
  PrefillPlan p;
  p.num_seqs = num_seqs;
  p.total_tokens = total_tokens;
  p.num_v_heads = num_v_heads;
  if (num_seqs <= 0) return p;
  p.seg_len = pick_seg_len(total_tokens, num_v_heads);
  // sum_i max(1, ceil(L_i / s)) <= N + T / s; segments that are not the last of
  // their sequence are full, so there are at most T / s of them.
  p.max_segments = num_seqs + total_tokens / p.seg_len;
  p.max_maps = total_tokens / p.seg_len;
  const size_t DD = (size_t)kD * kD * sizeof(float);
  size_t off = 0;
  p.off_table = off;
  off = align256(off + sizeof(int32_t) * 16 + sizeof(SegInfo) * (size_t)p.max_segments +
                 sizeof(int32_t) * (size_t)(p.max_maps + 1));
  if (p.max_maps > 0) {
    p.off_maps = off;
    off = align256(off + 2 * DD * (size_t)p.max_maps * num_v_heads);
    p.off_start = off;
    off = align256(off + DD * (size_t)p.max_segments * num_v_heads);
  }
  p.workspace_bytes = off;
  return p;
}

template <typename T>
static hipError_t launch_typed(const PrefillPlan &plan, PrefillArgs args, const int32_t *cu,
                               int N, int64_t Ttot, void *conv_out, hipStream_t stream,
                               PrefillTiming *tm) {
  const int Hv = args.Hv;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e;
    e = hipFuncSetAttribute((const void *)chunk_kernel<T, kFull>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void *)chunk_kernel<T, kMapA>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void *)chunk_kernel<T, kMapB>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  auto mark = [&](int slot) {  // event after kernel slot-1 (slot 0 = start)
    if (tm) (void)hipEventRecord(tm->ev[slot], stream);
  };
  if (tm) for (int i = 0; i < kTimedKernels; ++i) tm->ran[i] = false;
  if (tm) tm->ran[0] = true;  // the segment table was launched by the caller
  mark(1);
  if (plan.max_maps > 0) {
    dim3 g1((unsigned)(plan.max_maps * Hv));
    hipLaunchKernelGGL((chunk_kernel<T, kMapA>), g1, dim3(kThreads), kLdsBytes, stream, args);
    mark(2);
    hipLaunchKernelGGL((chunk_kernel<T, kMapB>), g1, dim3(kThreads), kLdsBytes, stream, args);
    mark(3);
    dim3 g2((unsigned)(plan.max_segments * Hv * 8));
    hipLaunchKernelGGL(combine_kernel, g2, dim3(256), 0, stream, args.segs, args.hdr,
                       args.init_state, (const float *)args.maps, args.starts, Hv);
    mark(4);
    if (tm) tm->ran[1] = tm->ran[2] = tm->ran[3] = true;
  } else {
    mark(2);
    mark(3);
    mark(4);
  }
  dim3 g3((unsigned)(plan.max_segments * Hv));
  hipLaunchKernelGGL((chunk_kernel<T, kFull>), g3, dim3(kThreads), kLdsBytes, stream, args);
  mark(5);
  if (tm) tm->ran[4] = true;
  if (conv_out) {
    const int64_t n = (int64_t)N * args.Cc;
    hipLaunchKernelGGL((conv_out_kernel<T>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       stream, cu, N, Ttot, (const T *)args.q, (const T *)args.k,
                       (const T *)args.v, (const T *)args.conv_in, (T *)conv_out, args.Hk,
                       args.Hv, args.Cc);
    if (tm) tm->ran[5] = true;
  }
  mark(6);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillPlan &plan, const void *q, const void *k, const void *v,
                          const float *a, const float *b, const void *z, const gdn_params &p,
                          const float *init_state, const int32_t *cu_seqlens, int32_t num_seqs,
                          int64_t total_tokens, const void *conv_state_in, void *o,
                          float *final_state, void *conv_state_out, void *workspace,
                          hipStream_t stream, PrefillTiming *tm) {
  unsigned char *ws = (unsigned char *)workspace;
  if (tm) (void)hipEventRecord(tm->ev[0], stream);
  int32_t *hdr = (int32_t *)(ws + plan.off_table);
  SegInfo *segs = (SegInfo *)(ws + plan.off_table + 16 * sizeof(int32_t));
  int32_t *map_seg = (int32_t *)(segs + plan.max_segments);
  hipLaunchKernelGGL(segment_table_kernel, dim3(1), dim3(1024), 0, stream, cu_seqlens, num_seqs,
                     total_tokens, plan.seg_len, plan.max_segments, plan.max_maps, segs, hdr,
                     map_seg);
  PrefillArgs A;
  A.q = q; A.k = k; A.v = v; A.z = z; A.a = a; A.b = b;
  A.conv_w = p.conv_weight; A.A_log = p.A_log; A.dt_bias = p.dt_bias; A.norm_w = p.norm_weight;
  A.q_scale = p.q_scale; A.l2_eps = p.l2_eps; A.rms_eps = p.rms_eps;
  A.init_state = init_state; A.conv_in = conv_state_in; A.o = o; A.final_state = final_state;
  A.segs = segs; A.hdr = hdr; A.map_seg = map_seg;
  A.maps = plan.max_maps > 0 ? (float *)(ws + plan.off_maps) : nullptr;
  A.starts = plan.max_maps > 0 ? (float *)(ws + plan.off_start) : nullptr;
  A.Hk = p.num_qk_heads; A.Hv = p.num_v_heads;
  A.Cc = 2LL * p.num_qk_heads * kD + (int64_t)p.num_v_heads * kD;
  const char *ev = getenv("GDN_PRECISE_ALL");
  A.precise_all = (ev && ev[0] == '1') ? 1 : 0;
  if (p.act_dtype == GDN_BF16)
    return launch_typed<bf16_t>(plan, A, cu_seqlens, num_seqs, total_tokens, conv_state_out,
                                stream, tm);
  return launch_typed<float>(plan, A, cu_seqlens, num_seqs, total_tokens, conv_state_out, stream,
                             tm);
}

}  // namespace gdn
