// gdn_attention.hip -- the hybrid's gated full-attention mixer on gfx950.
//
// Every fourth layer of the hybrid is softmax attention with grouped queries
// ("Qwen3-Next 80B-A3B" field guide, cutaway 03: 16 query heads share 2 key/value
// heads, head dim 256; RoPE on the first 64 dims; QK-Norm; a learned sigmoid output
// gate.  "Qwen3.8-Flash-Next" model card, attention entries: per-head RMSNorm of q and
// k before RoPE, a rotated and a position-free part of each head, the output times the
// sigmoid of a gate):
//   q^ = RoPE(RMSNorm(q) w_q),  k^ = RoPE(RMSNorm(k) w_k)   (positions from 0 per sequence)
//   o  = softmax_causal(q^ k^T * scale) v * sigmoid(gate),  q head h -> kv head h / (Hq/Hkv)
//
// Two kernels:
//   qk_prep_kernel   one pass over q and k: RMSNorm, weight, rotate-half RoPE of the
//                    first rotary_dim dims (angle in revolutions from an fp64 frequency
//                    table, reduced to [-1/2, 1/2] in fp64 before the hardware sine and
//                    cosine) -> fp16 q^, k^ in the workspace;
//   attention_kernel one workgroup = 4 waves of 32 queries each (up to four q heads of
//                    one kv head share it), keys in tiles of 32 through double-buffered
//                    LDS.  It computes S^T = K^ Q^T and O^T = V^T P^T on 32x32x16 MFMA,
//                    so a query is a column of both: its lane holds its softmax
//                    statistics, and P^T (C layout of S^T) is already the B operand of
//                    the second product (k slots in the permuted order the A operand V^T
//                    reads).  Online softmax in base 2; the next tile's scores are formed
//                    while the current tile's softmax runs.
#include "gdn_attention.h"
#include "gdn_device.h"
#include "gdn_launch.h"

#include <algorithm>
#include <cmath>

namespace gdn {

// Set by a call whose cu_seqlens table is invalid; read and cleared by
// take_attention_error().
__device__ int g_attn_bad_cu = 0;

namespace {

typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kAD = 256;          // head dim the kernels are built for

// Raw buffer over [base, base + bytes): loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int64_t bytes) {
  const int n = bytes > INT32_MAX ? INT32_MAX : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
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

// RoPE frequencies in revolutions per position: rev[i] = theta^(-2i/rotary_dim) / (2 pi),
// formed on the host in fp64 (passed by value with the kernel arguments).
struct RopeTable {
  double rev[kAD / 2];
};

// cu_seqlens tables up to this many entries are searched in LDS
constexpr int kCuLds = 1024;

// 256 threads = 8 rows of 256 at a time (32 threads x 8 dims each), over a grid-stride
// loop; rows are ordered token-major, q heads then kv heads.  The next row's input is
// loaded before the current one is processed, the norm weights once per thread, and a
// short cu_seqlens table is searched in LDS.
__global__ void __launch_bounds__(256)
qk_prep_kernel(const bf16_t *__restrict__ q, const bf16_t *__restrict__ k,
               const int32_t *__restrict__ cu, int N, int T, int Hq, int Hkv,
               const float *__restrict__ wq, const float *__restrict__ wk, int rot,
               RopeTable tab, float eps, int *__restrict__ bad_word,
               _Float16 *__restrict__ qh, _Float16 *__restrict__ kh) {
  __shared__ int s_cu[kCuLds];
  const bool cu_lds = cu && N < kCuLds;
  if (cu_lds)
    for (int i = threadIdx.x; i <= N; i += blockDim.x) s_cu[i] = cu[i];
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
  __syncthreads();
  const int H = Hq + Hkv;
  const int rows = T * H;  // below 2^27 (checked on the host)
  const int j = threadIdx.x & 31;  // dims 8j .. 8j + 7
  float wqj[8], wkj[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    wqj[e] = wq ? wq[8 * j + e] : 1.0f;
    wkj[e] = wk ? wk[8 * j + e] : 1.0f;
  }
  const int half = rot >> 1, sh = half >> 3;
  const bool rot_lane = 8 * j < rot, lo = 8 * j < half;
  const int partner = lo ? j + sh : j - sh;  // the lane holding this lane's RoPE pair
  auto src_of = [&](int row) {
    const int t = row / H, hh = row - t * H;
    return hh < Hq ? q + ((int64_t)t * Hq + hh) * kAD : k + ((int64_t)t * Hkv + hh - Hq) * kAD;
  };
  const int stride = gridDim.x * 8;
  int row = blockIdx.x * 8 + (threadIdx.x >> 5);
  if (row >= rows) return;  // uniform per 32-lane row group
  uint4 raw = *reinterpret_cast<const uint4 *>(src_of(row) + 8 * j);
  for (; row < rows; row += stride) {
    const uint4 cur = raw;
    if (row + stride < rows) raw = *reinterpret_cast<const uint4 *>(src_of(row + stride) + 8 * j);
    const int t = row / H, hh = row - t * H;
    const bool isq = hh < Hq;
    const uint32_t rw[4] = {cur.x, cur.y, cur.z, cur.w};
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
    for (int e = 0; e < 8; ++e) y[e] = x[e] * inv * (isq ? wqj[e] : wkj[e]);
    // rotate-half RoPE on dims < rot: dim d < rot/2 pairs with d + rot/2 (8-dim groups
    // rot/16 apart); every lane takes part in the exchange, only rotary lanes use it
    float pr[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pr[e] = __shfl(y[e], (int)(threadIdx.x & 32) + (partner & 31), 64);
    if (rot_lane) {
      int sbeg = 0;
      if (cu_lds) {
        int a = 0, b = N;  // s_cu[a] <= t < s_cu[b]
        while (b - a > 1) {
          const int mid = (a + b) >> 1;
          if (s_cu[mid] <= t) a = mid;
          else b = mid;
        }
        sbeg = s_cu[a];
      } else {
        sbeg = seq_begin(cu, N, t);
      }
      const int pos = t - sbeg;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = (lo ? 8 * j : 8 * j - half) + e;  // frequency index
        // angle in revolutions, pos * theta^(-2i/rot) / (2 pi), reduced to [-1/2, 1/2]
        // in fp64; the hardware sine and cosine take revolutions
        double rv = (double)pos * tab.rev[i];
        rv -= rint(rv);
        const float sn = __builtin_amdgcn_sinf((float)rv), cs = __builtin_amdgcn_cosf((float)rv);
        y[e] = lo ? y[e] * cs - pr[e] * sn : y[e] * cs + pr[e] * sn;
      }
    }
    _Float16 *dst = isq ? qh + ((int64_t)t * Hq + hh) * kAD : kh + ((int64_t)t * Hkv + hh - Hq) * kAD;
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    h8 out;
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (_Float16)y[e];
    *reinterpret_cast<h8 *>(dst + 8 * j) = out;
  }
}

// Key tiles of 32 through double-buffered LDS: K^ [32 keys][264] fp16 and V^T [256 dims][36
// keys] bf16 (the pads spread the MFMA operand reads over all banks).
constexpr int kKT = 32;
constexpr int kKsS = kAD + 8;
constexpr int kVtS = kKT + 4;
constexpr int kKBuf = kKT * kKsS;          // fp16 elements per K^ buffer
constexpr int kVBuf = kAD * kVtS;          // bf16 elements per V^T buffer
constexpr size_t kAttnLds = 2 * (size_t)kKBuf * 2 + 2 * (size_t)kVBuf * 2;
static_assert(kAttnLds <= 160 * 1024, "LDS budget");

__device__ __forceinline__ f32x16 mfma32h(u16x8 a, u16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32b(u16x8 a, u16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// One workgroup = 4 waves = hpb query heads of one kv head x qpb blocks of 32 queries
// (hpb * qpb <= 4; waves past that only help load the tiles).  Each wave owns 32 queries
// of one head: S^T [keys][32 queries] = K^ Q^T and O^T [256 dims][32 queries] += V^T P^T
// on 32x32x16 MFMA, so a lane holds one query's column (its softmax statistics) and P^T
// in C layout is already the B operand of the second product.  The running max m is
// only raised when a tile's max exceeds it by more than 8 (base 2), so O is rescaled
// rarely and p <= 2^8.
__global__ void __launch_bounds__(256, 1)
attention_kernel(const _Float16 *__restrict__ qh, const _Float16 *__restrict__ kh,
                 const bf16_t *__restrict__ v, const bf16_t *__restrict__ gate,
                 const int32_t *__restrict__ cu, int N, int T, int Hq, int Hkv, int hpb,
                 int qpb, float scale2, const int *__restrict__ bad_word,
                 bf16_t *__restrict__ o) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  _Float16 *const sK = reinterpret_cast<_Float16 *>(smem);
  bf16_t *const sVt = reinterpret_cast<bf16_t *>(smem + 2 * (size_t)kKBuf * 2);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 31, lh = lane >> 5;
  const int r = Hq / Hkv, ng = r / hpb;
  // ids 8 apart go to the same XCD: the ng head groups of one (kv head, query block)
  // get ids 8 apart, so their shared K^ and V tiles are fetched into one L2
  const int bid = blockIdx.x, x = bid & 7, yb = bid >> 3;
  const int member = yb % ng, rest = (yb / ng) * 8 + x;
  const int span = 32 * qpb;
  const int nqb = (T + span - 1) / span;
  if (rest >= nqb * Hkv) return;
  if (bad_word && *bad_word) return;  // invalid cu_seqlens: o is left unwritten
  // the last query blocks see the most keys: they are dispatched first
  const int qb = nqb - 1 - rest / Hkv, kvh = rest % Hkv;
  const int t0 = qb * span;
  const bool active = wave < hpb * qpb;
  const int h = kvh * r + member * hpb + (active ? wave % hpb : 0);
  const int t0w = t0 + 32 * (active ? wave / hpb : 0);   // the wave's first query
  const int tq = t0w + ln;                               // this lane's query
  const bool qvalid = active && tq < T;
  const int tqc = min(tq, T - 1);
  // sequence starts (clamped, so that no table can send an access out of bounds)
  const int sb = min(max(seq_begin(cu, N, tqc), 0), tqc);
  const int kstart = min(max(seq_begin(cu, N, t0), 0), t0);
  const int kend = min(t0 + span - 1, T - 1);
  // wave-uniform key range that needs no mask: [sb_hi, t0w]
  const int tlast = min(t0w + 31, T - 1);
  const int sb_hi = min(max(seq_begin(cu, N, tlast), 0), tlast);
  const int wave_kend = active && t0w < T ? tlast : -1;

  // Q^ fragments (B operand): lane holds dims 16c + 8lh .. + 7 of its query
  u16x8 qf[16];
#pragma unroll
  for (int c = 0; c < 16; ++c)
    qf[c] = *reinterpret_cast<const u16x8 *>(qh + ((int64_t)tqc * Hq + h) * kAD + 16 * c + 8 * lh);
  // Q^ lives in AGPRs (the MFMA reads its B operand from there), which leaves the
  // VGPRs to O, the scores and the operand reads in flight
#pragma unroll
  for (int c = 0; c < 16; ++c) asm volatile("" : "+a"(qf[c]));

  f32x16 oacc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m = -INFINITY, l = 0.f;

  // Tile staging: K^ chunk c = tid + 256 i (key c / 32, dims 8 (c % 32)); V keys
  // 4 kq .. + 3 (kq = tid % 8) at dims 8 dc .. + 7 (dc = tid / 8).  Buffers start at
  // the tile's first key, so keys past T read as zero.
  //
  // Software pipeline: in iteration it a wave forms the scores of tile it + 1 on MFMA
  // while its VALU runs the softmax of tile it, then O^T += V^T P^T of tile it.  So K^
  // runs two tiles ahead of V: at the start of iteration it, K^ buffers hold tiles it and
  // it + 1 and V^T buffer it & 1 holds tile it; during it the block stores K^(it + 2)
  // (over K^(it), last read in iteration it - 1) and V(it + 1) (over V(it - 1)).
  typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
  i32x4 gk[4], gv[4];
  const int64_t key_bytes = (int64_t)Hkv * kAD * 2;
  auto gload_k = [&](int k0) {
    const auto rk = rsrc(kh + ((int64_t)k0 * Hkv + kvh) * kAD, (int64_t)(T - k0) * key_bytes);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      gk[i] = __builtin_amdgcn_raw_buffer_load_b128(
          rk, (uint32_t)((c >> 5) * key_bytes + 16 * (c & 31)), 0, 0);
    }
  };
  auto gload_v = [&](int k0) {
    const auto rv = rsrc(v + ((int64_t)k0 * Hkv + kvh) * kAD, (int64_t)(T - k0) * key_bytes);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      gv[e] = __builtin_amdgcn_raw_buffer_load_b128(
          rv, (uint32_t)((4 * (tid & 7) + e) * key_bytes + 16 * (tid >> 3)), 0, 0);
  };
  auto lstore_k = [&](int buf) {
    _Float16 *k_ = sK + buf * kKBuf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      *reinterpret_cast<i32x4 *>(k_ + (c >> 5) * kKsS + 8 * (c & 31)) = gk[i];
    }
  };
  auto lstore_v = [&](int buf) {
    bf16_t *v_ = sVt + buf * kVBuf;
    const int dc = tid >> 3, kq = tid & 7;
#pragma unroll
    for (int e = 0; e < 8; ++e) {  // dim 8 dc + e of keys 4 kq .. + 3
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      const int w = e >> 1;
      const uint32_t lo = __builtin_amdgcn_perm((uint32_t)gv[1][w], (uint32_t)gv[0][w], sel);
      const uint32_t hi = __builtin_amdgcn_perm((uint32_t)gv[3][w], (uint32_t)gv[2][w], sel);
      *reinterpret_cast<uint2 *>(v_ + (8 * dc + e) * kVtS + 4 * kq) = make_uint2(lo, hi);
    }
  };
  const int ntiles = (kend - kstart) / kKT + 1;
  // loads issued at the top of iteration it and stored at its bottom
  auto loads = [&](int it) {
    if (it + 2 < ntiles) gload_k(kstart + (it + 2) * kKT);
    if (it + 1 < ntiles) gload_v(kstart + (it + 1) * kKT);
  };
  auto stores = [&](int it) {
    if (it + 2 < ntiles) lstore_k(it & 1);
    if (it + 1 < ntiles) lstore_v((it + 1) & 1);
  };

  // raw scores S^T of the tile in K^ buffer buf (lane: keys 8 (i / 4) + 4 lh + i % 4)
  auto scores = [&](int buf) {
    const _Float16 *k_ = sK + buf * kKBuf;
    f32x16 st;
#pragma unroll
    for (int i = 0; i < 16; ++i) st[i] = 0.f;
    // operand reads in batches of 8 ahead of their products
#pragma unroll
    for (int c0 = 0; c0 < 16; c0 += 8) {
      u16x8 a[8];
#pragma unroll
      for (int c = 0; c < 8; ++c)
        a[c] = *reinterpret_cast<const u16x8 *>(k_ + ln * kKsS + 16 * (c0 + c) + 8 * lh);
#pragma unroll
      for (int c = 0; c < 8; ++c) st = mfma32h(a[c], qf[c0 + c], st);
    }
    return st;
  };
  // Online softmax of the tile at k0 with raw scores st, in two parts: `limit` masks
  // the scores and updates the reference max (its branches stay ahead of the next
  // tile's score products), `accumulate` forms p and O^T += V^T P^T.
  auto limit = [&](f32x16 &st, int k0) {
    const bool full = k0 >= sb_hi && k0 + kKT - 1 <= t0w;
    if (!full) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + 8 * (i >> 2) + 4 * lh + (i & 3);
        const bool ok = qvalid && key >= sb && key <= tq;
        st[i] = ok ? st[i] : -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, st[i]);
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                       false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * scale2;
    }
    // raise the reference max only when this tile exceeds it by more than 8
    const bool raise = mx > m + 8.0f;
    if (__builtin_amdgcn_ballot_w64(raise)) {
      const float al = raise ? exp2f(m - mx) : 1.0f;  // m = -inf: al = 0 (O, l are 0)
      if (raise) m = mx;
      l *= al;
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= al;
    }
  };
  auto accumulate = [&](f32x16 st, int buf) {
    const bf16_t *v_ = sVt + buf * kVBuf;
    const float mu = m == -INFINITY ? 0.f : m;  // no key yet: every p is 0
    // p = 2^(scale2 s - mu) <= 2^8; masked scores are -inf and give 0
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      st[i] = __builtin_amdgcn_exp2f(fmaf(st[i], scale2, -mu));
      ps += st[i];
    }
    l += ps;  // this lane's half of the keys; the halves are added at the end
    // O^T += V^T P^T over two 16-key chunks: slot 8 lh + j <-> key 16 kc + 4 lh + j
    // (j < 4) and 16 kc + 8 + 4 lh + j - 4 (j >= 4), the lane's C-layout values
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const int i0 = 8 * kc;
      const u16x8 pb = __builtin_bit_cast(
          u16x8, make_uint4(pk_bf16(st[i0], st[i0 + 1]), pk_bf16(st[i0 + 2], st[i0 + 3]),
                            pk_bf16(st[i0 + 4], st[i0 + 5]), pk_bf16(st[i0 + 6], st[i0 + 7])));
      u16x8 a[8];
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const bf16_t *row = v_ + (32 * db + ln) * kVtS + 16 * kc + 4 * lh;
        const uint2 lo = *reinterpret_cast<const uint2 *>(row);
        const uint2 hi = *reinterpret_cast<const uint2 *>(row + 8);
        a[db] = __builtin_bit_cast(u16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
      }
#pragma unroll
      for (int db = 0; db < 8; ++db) oacc[db] = mfma32b(a[db], pb, oacc[db]);
    }
  };

  // Every wave takes part in loading all of the block's tiles; it computes only those
  // holding a key in [its first query's sequence start, its last query]: tiles
  // it_lo .. it_hi.  Separate loops keep the tile-skip decisions out of the loop that
  // carries O.
  const int sb_lo = min(max(seq_begin(cu, N, min(t0w, T - 1)), 0), t0w);
  int it_lo = __builtin_amdgcn_readfirstlane(wave_kend >= 0 ? (sb_lo - kstart) / kKT : ntiles);
  const int it_hi = __builtin_amdgcn_readfirstlane(wave_kend >= 0 ? (wave_kend - kstart) / kKT : -1);
  it_lo = min(max(it_lo, 0), ntiles);
  gload_k(kstart);
  gload_v(kstart);
  lstore_k(0);
  lstore_v(0);
  if (ntiles > 1) {
    gload_k(kstart + kKT);
    lstore_k(1);
  }
  __syncthreads();
  f32x16 scur;
  if (it_lo == 0 && it_hi >= 0) scur = scores(0);
  __syncthreads();  // K^(0) is read before iteration 0 stores K^(2) over it
  int it = 0;
  for (; it + 1 < it_lo; ++it) {  // tiles before the wave's range
    loads(it);
    stores(it);
    __syncthreads();
  }
  if (it + 1 == it_lo && it_lo <= it_hi) {  // the wave's first scores
    loads(it);
    scur = scores((it + 1) & 1);
    stores(it);
    __syncthreads();
    ++it;
  }
  for (; it < it_hi; ++it) {  // scores of it + 1 on MFMA beside the softmax of it
    loads(it);
    limit(scur, kstart + it * kKT);
    const f32x16 snext = scores((it + 1) & 1);
    accumulate(scur, it & 1);
    scur = snext;
    stores(it);
    __syncthreads();
  }
  if (it == it_hi) {  // the wave's last tile
    loads(it);
    limit(scur, kstart + it * kKT);
    accumulate(scur, it & 1);
    stores(it);
    __syncthreads();
    ++it;
  }
  for (; it < ntiles; ++it) {  // tiles after the wave's range
    loads(it);
    stores(it);
    __syncthreads();
  }

  // epilogue: lane holds dims 32 db + 8 (i / 4) + 4 lh + i % 4 of its query; o / l * sigmoid(gate)
  if (!qvalid) return;
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l), false,
                                                     false);
    l = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  const float il = l > 0.f ? 1.0f / l : 0.f;
  const int64_t base = ((int64_t)tq * Hq + h) * kAD;
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = 32 * db + 8 * g4 + 4 * lh;
      const uint2 gw = *reinterpret_cast<const uint2 *>(gate + base + d);
      const float g[4] = {__uint_as_float(gw.x << 16), __uint_as_float(gw.x & 0xFFFF0000u),
                          __uint_as_float(gw.y << 16), __uint_as_float(gw.y & 0xFFFF0000u)};
      float val[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) val[i] = oacc[db][4 * g4 + i] * il * sigmoidf_(g[i]);
      *reinterpret_cast<uint2 *>(o + base + d) = make_uint2(pk_bf16(val[0], val[1]),
                                                            pk_bf16(val[2], val[3]));
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
  RopeTable tab{};
  for (int i = 0; i < rotary_dim / 2; ++i)
    tab.rev[i] = std::pow((double)theta, -2.0 * i / rotary_dim) / 6.283185307179586;
  // a few resident workgroups per CU, each looping over rows
  const int64_t prep_blocks = std::min<int64_t>((rows + 7) / 8, 256 * 5);
  hipLaunchKernelGGL(qk_prep_kernel, dim3((unsigned)prep_blocks), dim3(256), 0, stream,
                     (const bf16_t *)q, (const bf16_t *)k, cu, N, (int)T, Hq, Hkv, wq, wk,
                     rotary_dim, tab, eps, bad_word, qh, kh);
  // heads per workgroup: the largest divisor of Hq / Hkv up to 4; the rest of the four
  // waves take further 32-query blocks of the same heads
  const int r = Hq / Hkv;
  int hpb = 1;
  for (int d = 4; d >= 1; --d)
    if (r % d == 0) { hpb = d; break; }
  const int qpb = 4 / hpb;
  const int64_t span = 32 * qpb;
  const int64_t nqb = (T + span - 1) / span;
  const int64_t pairs = nqb * Hkv;
  const int64_t blocks = (pairs + 7) / 8 * 8 * (r / hpb);
  static std::atomic<uint64_t> lds_set{0};
  if (hipError_t e = ensure_lds_limit((const void *)attention_kernel, (int)kAttnLds, lds_set);
      e != hipSuccess)
    return e;
  hipLaunchKernelGGL(attention_kernel, dim3((unsigned)blocks), dim3(256), kAttnLds, stream,
                     (const _Float16 *)qh, (const _Float16 *)kh, (const bf16_t *)v,
                     (const bf16_t *)gate, cu, N, (int)T, Hq, Hkv, hpb, qpb,
                     scale * 1.4426950408889634f, (const int *)bad_word, (bf16_t *)o);
  return hipGetLastError();
}

}  // namespace gdn
