// gdn_prefill.hip -- chunked prefill of the Gated DeltaNet mixer on gfx950.
//
// Method (rows = tokens of one 32-token chunk, H = S^T [dk][dv] the state the
// chunk enters with, g = log alpha, G = chunk-local cumsum of g, gamma = e^G):
//   L[i][j] = beta_i e^{G_i-G_j} (k_i . k_j)  (j < i)      T = (I + L)^-1
//   W       = T diag(beta gamma) K                         Utilde = T diag(beta) V
//   U       = Utilde - W H                                 ("v_new")
//           = T (diag(beta) V - diag(beta gamma) K H)      (the form computed: one solve)
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
// Precision plan (fp32 accumulation, fp32 state): every product takes fp16
// operands.  q and k are unit-norm (q_scale multiplies o at the end), |L| <= 1 and
// the entries of each (I + L_bb)^-1 stay below 2^15; the right-hand side of the
// triangular solve is scaled by a power of two per wave, and the state by another
// one (sigma, with a tracked bound that keeps |sigma H| below 2^14), so every fp16
// operand is in range.  The identity part of the solve (its right-hand side) and the
// diagonal of M U are applied in fp32.  Powers of two are exact: o and the final
// state are divided by them at the end.
//
// Work decomposition: a workgroup runs NH v heads of one q/k head and one segment,
// 4 waves per v head; wave role w owns value columns 32w..32w+31 of its head's state
// in MFMA accumulators.  NH = 2 (the v heads of a q/k head pair up): 8 waves, one
// workgroup per compute unit, and the q/k prologue (conv, SiLU, L2 norm, the fp16 q,
// k and K^T tiles) is computed once for both heads.  NH = 1: 4 waves, two
// workgroups per compute unit (~60 KB of LDS and <= 256 VGPRs each), so that one's
// VALU-bound prologue and epilogue overlap the other's LDS- and MFMA-bound chain.
// Long sequences are cut into segments: pass 1 computes each non-final segment's
// affine map H -> A H + B (the same chunk loop run on the columns of A = I and
// B = 0, NH = 1), pass 2 chains the maps into segment start states, pass 3 runs the
// full chunk loop of every segment from its start state.
#include "gdn_device.h"
#include "gdn_prefill_plan.h"
#include "gdn_launch.h"

namespace gdn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(u16x8 a, u16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
// the same product with fp16 operands (same lane layout)
__device__ __forceinline__ f32x4 mfma16h(u16x8 a, u16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// Raw buffer over [base, base + bytes) (uniform): loads past the end return 0
// and stores past it are dropped, so ragged tails need no per-lane clamps.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ rsrc_t buf(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}
template <typename T> struct BufIO;
template <> struct BufIO<bf16_t> {
  static __device__ __forceinline__ uint32_t bits(rsrc_t r, uint32_t off) {
    return (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
  }
  static __device__ __forceinline__ void store(rsrc_t r, uint32_t off, float x) {
    __builtin_amdgcn_raw_buffer_store_b16(f2bf(x), r, off, 0, 0);
  }
};
// 8 consecutive outputs of one row, rounded to T, as 16-byte buffer stores
template <typename T> struct OutRow;
template <> struct OutRow<bf16_t> {
  static __device__ __forceinline__ void store(rsrc_t r, uint32_t off, const float *x) {
    const i32x4 w = {(int)pk_bf16(x[0], x[1]), (int)pk_bf16(x[2], x[3]), (int)pk_bf16(x[4], x[5]),
                     (int)pk_bf16(x[6], x[7])};
    __builtin_amdgcn_raw_buffer_store_b128(w, r, off, 0, 0);
  }
};
template <> struct OutRow<float> {
  static __device__ __forceinline__ void store(rsrc_t r, uint32_t off, const float *x) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, f32x4{x[0], x[1], x[2], x[3]}),
                                           r, off, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, f32x4{x[4], x[5], x[6], x[7]}),
                                           r, off + 16, 0, 0);
  }
};
template <> struct BufIO<float> {
  static __device__ __forceinline__ uint32_t bits(rsrc_t r, uint32_t off) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  }
  static __device__ __forceinline__ void store(rsrc_t r, uint32_t off, float x) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, off, 0, 0);
  }
};

// fp32 -> fp16 bits (round to nearest even)
__device__ __forceinline__ bf16_t f2h(float x) { return __builtin_bit_cast(bf16_t, (_Float16)x); }
// biased exponent field of |x| (0 for zero and denormals, 255 for Inf and NaN)
__device__ __forceinline__ int exp_bits(float x) {
  return (int)((__float_as_uint(x) >> 23) & 0xFF);
}

// (fp16 in the low / high half of w) * b in one v_fma_mix_f32 (the fp16 value is
// widened exactly, the product rounded once, as (float)h * b)
__device__ __forceinline__ float mul_lo_h(uint32_t w, float b) {
  float d;
  asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[0,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(w), "v"(b));
  return d;
}
__device__ __forceinline__ float mul_hi_h(uint32_t w, float b) {
  float d;
  asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(w), "v"(b));
  return d;
}

// 2^e as a float, e in [-126, 127]
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

__device__ __forceinline__ u16x8 cat4(u16x4 x, u16x4 y) {
  return u16x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
}

// --------------------------------------------------------------------- LDS
// A workgroup runs NH v heads of one q/k head with 4 waves per v head.  NH = 1: two
// workgroups share a compute unit (LDS <= 80 KB and <= 256 VGPRs each), so one's
// VALU-heavy prologue/epilogue overlaps the other's LDS- and MFMA-heavy chain.
// NH = 2: one 8-wave workgroup per compute unit; the q/k prologue (conv, SiLU, L2
// norm, the fp16 tiles) is computed once for both v heads.
constexpr int kThreads = 256;  // 4 waves per v head
constexpr int kWaves = 4;
constexpr int kRowS = 136;     // bf16 row stride of [32 tok][128 d] tiles (272 B)
constexpr int kTokS = 36;      // 16-bit row stride of the [128 d][32 tok] K^T tile (72 B)
constexpr int kSqS = 36;       // bf16 row stride of [32][32] tiles (M, -L)
constexpr int kVtS = 36;       // fp32 row stride of the [128 dv][32 tok] V^T tile (144 B)
constexpr float kConvScale = -1.4426950408889634f;  // -log2(e), folded into the conv taps
constexpr int kConvGS = 36;  // fp32 stride of 8 channels x 4 taps (padded: no bank conflicts)
// Per-token gate vectors of a chunk, two buffers (chunk parity): the next chunk's
// are written while this chunk's are in use.  Vector k of a buffer starts at float
// k * kChunk: beta, G (cumsum of g), gamma = e^G, beta gamma, e^{G_C - G},
// beta / kConvScale (multiplies scaled v).
enum { GB_BETA = 0, GB_G, GB_GAM, GB_BG, GB_DEC, GB_BV, GB_N };
constexpr int kGateN = GB_N * kChunk;  // floats per buffer
constexpr int kTdS = 24;               // bf16 row stride of (T_bb - I) blocks
constexpr int kOS = 132;               // fp32 row stride of the [32 tok][128] o tile
constexpr int kMaxSegChunks = 256;     // segments hold at most 8192 tokens

// Byte offsets.  Shared by the workgroup's v heads: the fp16 unit-norm q and k rows,
// the fp16 K^T tile, the conv taps of q, k and every v head, the RMSNorm weight.  One
// block per v head: V^T (fp32; map mode's chunk sums reuse it before the chunk loop),
// M, the gate buffers, M's diagonal, -L and T_bb - I (regions of their own, so the
// waves that form them need not wait for the others' gram products), the o tile.
template <int NH> struct Lds {
  static constexpr int QF = 0;                           // fp16 q [32][136] (Q K^T, Q H)
  static constexpr int KF = QF + kChunk * kRowS * 2;     // fp16 k [32][136] (K K^T, Q K^T)
  static constexpr int KT = KF + kChunk * kRowS * 2;     // fp16 K^T [128 dk][32 tok]
  static constexpr int CONVW = KT + 128 * kTokS * 2;     // taps: q, k, then each v head
  static constexpr int NW = CONVW + (32 + 16 * NH) * kConvGS * 4;  // fp32 [128]
  static constexpr int HEAD = NW + kD * 4;               // first per-head block
  static constexpr int H_VT = 0;                         // fp32 V^T [128 dv][36]
  static constexpr int H_M = H_VT + 128 * kVtS * 4;      // fp16 [32][36] M, zero diagonal
  static constexpr int H_GATES = H_M + kChunk * kSqS * 2;
  static constexpr int H_MDIAG = H_GATES + 2 * kGateN * 4;
  static constexpr int H_LO = H_MDIAG + kChunk * 4;      // fp16 [32][36] -L (strictly lower)
  static constexpr int H_TD = H_LO + kChunk * kSqS * 2;  // fp16 [2][16][24] T_bb - I
  static constexpr int H_O = H_TD + 2 * 16 * kTdS * 2;   // fp32 [32 tok][132] o tile
  static constexpr int H_BYTES = H_O + kChunk * kOS * 4;
  static constexpr int BYTES = HEAD + NH * H_BYTES;
  static_assert(HEAD % 16 == 0 && H_BYTES % 16 == 0 && H_TD % 16 == 0, "16-byte tiles");
  static_assert(kMaxSegChunks * 4 <= 128 * kVtS * 4, "chunk sums overflow the V^T region");
  static_assert(NH == 2 ? BYTES <= 160 * 1024 : 2 * BYTES <= 160 * 1024,
                "LDS budget: two 4-wave or one 8-wave workgroup per compute unit");
};
static_assert(kChunk == 32, "the tile code below is written for 32-token chunks");

enum Mode { kFull = 0, kMap = 1 };

// Set (to 1) by the segment table (or, for one sequence, by the kernels) when
// cu_seqlens is invalid; read and cleared by the host (gdn_check_device_errors).  One
// copy per device.
__device__ int g_prefill_bad_cu = 0;

// Segments of a sequence of len tokens: max(1, ceil(len / seg_len)).
__host__ __device__ __forceinline__ int seg_count(int len, int seg_len) {
  return len == 0 ? 1 : (len + seg_len - 1) / seg_len;
}
// Record of segment s of sequence seq = tokens [b, e): the chunks are spread evenly
// over the segments (the first nch % ns get one more), so every segment of a split
// sequence holds >= 4 full chunks.  first / firstmap: the global index of the
// sequence's first segment / map slot (the non-final segments take map slots in order).
__device__ __forceinline__ SegInfo seg_record(int seq, int b, int e, int s, int seg_len, int first,
                                              int firstmap) {
  const int len = e - b;
  const int ns = seg_count(len, seg_len), nch = (len + kChunk - 1) / kChunk;
  const int q = nch / ns, rem = nch % ns;
  SegInfo si;
  si.seq = seq;
  si.begin = b + kChunk * (s * q + min(s, rem));
  si.len = max(0, min(kChunk * (q + (s < rem ? 1 : 0)), e - si.begin));
  si.idx = s;
  si.nseg = ns;
  si.first = first;
  si.map = s < ns - 1 ? firstmap + s : -1;
  si.seq_begin = b;
  return si;
}

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
  const int32_t *seq_first;  // sequence -> index of its first segment
  const int32_t *order;      // full-pass unit -> segment index (longest segments first)
  float *maps;             // [max_maps][Hv][2][D][D]
  int32_t *map_zero;       // [max_maps][Hv]: 1 if the A map is zero (not stored)
  float *starts;           // [max_segments][Hv][D][D]
  int Hk, Hv;
  int64_t Cc;
  int gate;                // output gate: 0 SiLU(z), 1 sigmoid(z)
  // one sequence: no table is built, the kernels form each segment's record from
  // (seg_len, T) with seg_record; cu (cu_seqlens or NULL) is checked by every workgroup
  int one_seq, seg_len, T;
  const int32_t *cu;
};

// One sequence with a cu_seqlens table: it must read {0, T}.  A workgroup that finds
// otherwise flags the call (as the segment table does for longer tables) and exits.
__device__ __forceinline__ bool one_seq_table_bad(const int32_t *cu, int T) {
  if (!cu) return false;
  const bool bad = cu[0] != 0 || cu[1] != T;
  if (bad) g_prefill_bad_cu = 1;
  return bad;
}

// NC channels of one token as raw 32-bit words (bf16 pairs or fp32)
template <typename T, int NC>
struct RawN {
  static constexpr int W = NC * (int)sizeof(T) / 4;
  static_assert(W == 2 || W == 4 || W == 8, "row fragment of 8, 16 or 32 bytes");
  static __device__ __forceinline__ void load(uint32_t (&dst)[W], const T *p) {
    const uint32_t *q = reinterpret_cast<const uint32_t *>(p);
    if (W == 2) {
      const uint2 t = *reinterpret_cast<const uint2 *>(q);
      dst[0] = t.x; dst[1] = t.y;
    } else {
#pragma unroll
      for (int i = 0; i < W; i += 4) {
        const uint4 t = *reinterpret_cast<const uint4 *>(q + i);
        dst[i] = t.x; dst[i + 1] = t.y; dst[i + 2] = t.z; dst[i + 3] = t.w;
      }
    }
  }
  static __device__ __forceinline__ void load_buf(uint32_t (&dst)[W], rsrc_t r, uint32_t off) {
    if (W == 2) {
      const auto t = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
      dst[0] = t[0]; dst[1] = t[1];
    } else {
#pragma unroll
      for (int i = 0; i < W; i += 4) {
        const i32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, off + 4 * i, 0, 0);
        dst[i] = t.x; dst[i + 1] = t.y; dst[i + 2] = t.z; dst[i + 3] = t.w;
      }
    }
  }
  static __device__ __forceinline__ float get(const uint32_t (&w)[W], int c) {
    if (sizeof(T) == 4) return __uint_as_float(w[c]);
    const uint32_t word = w[c >> 1];
    return __uint_as_float((c & 1) ? (word & 0xFFFF0000u) : (word << 16));
  }
};

// Width-4 causal conv + SiLU of NT tokens x NC channels.  raw[r] holds the raw
// inputs of token tbase - 3 + r of the chunk; wv the NC x 4 taps (tap 3 = current
// token) pre-multiplied by kConvScale = -log2(e), so that the conv output a is
// -log2(e) u and SiLU(u) = u / (1 + e^-u) comes out as a / (1 + 2^a), i.e.
// scaled by kConvScale: the L2 norm of q and k absorbs the scale (and its
// sign), the beta that multiplies v in the right-hand side absorbs it for v.
// Tokens past the end of a partial chunk come out as finite values that never
// reach an output: their beta is 0, so their rows of L, W and Utilde (and
// hence U) are exactly zero, and their o rows are not stored.
template <typename T, int NT, int NC>
__device__ __forceinline__ void conv_silu_rows(const uint32_t (&raw)[NT + 3][RawN<T, NC>::W],
                                               const float *wv, float (&x)[NT][NC]) {
  float w[NC][4];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) {
    const f32x4 t = *reinterpret_cast<const f32x4 *>(wv + cc * 4);
    w[cc][0] = t.x; w[cc][1] = t.y; w[cc][2] = t.z; w[cc][3] = t.w;
  }
#pragma unroll
  for (int r = 0; r < NT; ++r) {
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) acc += w[cc][j] * RawN<T, NC>::get(raw[r + j], cc);
      x[r][cc] = acc * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(acc));
    }
  }
}

// fp16 B operand (K = 32) from two 16x16 C-layout tiles, each scaled by f: slot
// 8lg+j <-> row 4lg+j of tile a (j < 4), row 4lg+j-4 of tile b (j >= 4).  Any A
// operand paired with it reads its k index in the same order.
__device__ __forceinline__ u16x8 pack_h(const f32x4 &a, const f32x4 &b, float f = 1.0f) {
  const uint32_t w0 = pk_f16(a[0] * f, a[1] * f), w1 = pk_f16(a[2] * f, a[3] * f);
  const uint32_t w2 = pk_f16(b[0] * f, b[1] * f), w3 = pk_f16(b[2] * f, b[3] * f);
  return __builtin_bit_cast(u16x8, make_uint4(w0, w1, w2, w3));
}
// A operand row fragment in the permuted k order: cols c0+4lg..+3 and c1+4lg..+3
__device__ __forceinline__ u16x8 load_a_perm(const bf16_t *row, int c0, int c1, int lg) {
  return cat4(*reinterpret_cast<const u16x4 *>(row + c0 + 4 * lg),
              *reinterpret_cast<const u16x4 *>(row + c1 + 4 * lg));
}

// [row][tok] tiles over the chunk's 32 tokens (bf16 K^T hi/lo, fp32 V^T): the
// eight 4-token groups of a row are XOR-swizzled with bits 4..6 of the row.  The
// prologue writes rows 8 (K^T) or 16 (V^T) apart from neighbouring lanes, which
// the swizzle spreads over all banks; the MFMA reads take rows 16*rt + lane, for
// which the swizzle is the constant rt.
__device__ __forceinline__ int tok_swz(int row, int tok, int stride) {
  return row * stride + ((((tok >> 2) ^ (row >> 4)) & 7) << 2) + (tok & 3);
}
// Lane part of the K^T reads of rows 16*rt + ln, tokens 4lg..4lg+3 (half 0) and
// 16+4lg..16+4lg+3 (half 1): with lg < 4 the swizzled group is (lg ^ (rt & 3))
// plus a constant, so four lane bases cover every rt.
struct TokLane {
  int base[4];
  __device__ __forceinline__ TokLane(int ln, int lg) {
#pragma unroll
    for (int d = 0; d < 4; ++d) base[d] = ln * kTokS + 4 * (lg ^ d);
  }
  __device__ __forceinline__ int operator()(int rt, int half) const {
    return base[rt & 3] + 16 * rt * kTokS + 4 * (half ? 4 - (rt & 4) : (rt & 4));
  }
};
// A operand of K^T U: rows 16rt + ln, tokens in the permuted k order of pack_h
// (4lg .. +3, then 16 + 4lg .. +3)
__device__ __forceinline__ u16x8 load_a_tok(const bf16_t *tile, const TokLane &tl, int rt) {
  return cat4(*reinterpret_cast<const u16x4 *>(tile + tl(rt, 0)),
              *reinterpret_cast<const u16x4 *>(tile + tl(rt, 1)));
}

typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
// 16x16 operand with K = 16 in fp16, packed from a C-layout tile X (lane ln, lg
// holds rows 4lg..4lg+3 of column ln, which is the k order of the 16x16x16
// product): as a B operand this is X, as an A operand it is the transpose of X.
__device__ __forceinline__ f16x4_t h4(const f32x4 &x) {
  return __builtin_bit_cast(f16x4_t, make_uint2(pk_f16(x[0], x[1]), pk_f16(x[2], x[3])));
}
// c + A B with A = transpose of the tile packed in a, B = the tile packed in b
__device__ __forceinline__ f32x4 mm16(f16x4_t a, f16x4_t b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// Transpose of (I + L)^-1 for a strictly lower 16x16 block L, given the C-layout
// tiles of M = -L^T (mc) and of M^T = -L (mt).  L is nilpotent (L^16 = 0), so
// (I + L)^-1 = (I + N)(I + N^2)(I + N^4)(I + N^8) with N = -L; the transpose is
// the same product in M, and all factors commute.  |L_ij| <= 1 (beta <= 1, decay
// <= 1, unit-norm keys), so every power and partial product has entries below
// 2^15 and fits fp16; fp16 operands (11-bit significands) keep the products well
// below the bf16 rounding applied to T - I.
__device__ __forceinline__ f32x4 unit_lower_inverse_t(const f32x4 &mc, const f32x4 &mt, int ln,
                                                      int lg) {
  const f32x4 Z = {0.f, 0.f, 0.f, 0.f};
  const f16x4_t sm = h4(mc), smt = h4(mt);
  const f32x4 m2 = mm16(smt, sm, Z), m2t = mm16(sm, smt, Z);        // M^2, (M^2)^T
  const f16x4_t sm2 = h4(m2), sm2t = h4(m2t);
  const f32x4 m4 = mm16(sm2t, sm2, Z), m4t = mm16(sm2, sm2t, Z);    // M^4, (M^4)^T
  const f32x4 m8t = mm16(h4(m4), h4(m4t), Z);                       // (M^8)^T
  f32x4 t = mc;  // I + M
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (4 * lg + i == ln) t[i] += 1.0f;
  t = mm16(sm2t, h4(t), t);        // (I + M)(I + M^2)
  t = mm16(h4(m4t), h4(t), t);     // ... (I + M^4)
  return mm16(h4(m8t), h4(t), t);  // ... (I + M^8)
}

// ------------------------------------------------------------ chunk kernel
// MODE kFull: the whole mixer for one segment and NH v heads.  MODE kMap: the
// segment's affine map; blockIdx selects the A half (state columns of the
// identity) or the B half (columns of zero with the values written in).
template <typename T, int MODE, int NH>
__global__ void __launch_bounds__(kThreads * NH, 2 / NH) chunk_kernel(PrefillArgs P) {
  static_assert(NH == 1 || (NH == 2 && MODE == kFull), "two v heads per workgroup: full pass");
  typedef Lds<NH> L;
  constexpr int kTh = kThreads * NH;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  // Physical wave pw = tid / 64; head slot hh = pw / 4; wave = the role within the head
  // (state columns 32 wave.., gram tile, gates).  The second head's roles are rotated by
  // two, so that each SIMD (waves pw and pw + 4) holds one of the diagonal-tile waves
  // (roles 0, 1) and one of the others.
  int tid = threadIdx.x;
  int hh = 0, wave, lane = tid & 63;
  auto roles = [&]() {
    const int pw = __builtin_amdgcn_readfirstlane(tid >> 6);
    hh = NH == 2 ? pw >> 2 : 0;
    wave = NH == 2 ? (pw + 2 * hh) & 3 : pw;
  };
  roles();
  int ln = lane & 15, lg = lane >> 4;  // MFMA lane coordinates
  const int Hv = P.Hv, Hk = P.Hk;
  // Workgroup ids go round-robin over the 8 XCDs (each with its own L2).  The
  // r / NH workgroups that read the same q/k head get ids 8 apart, i.e. the same
  // XCD at nearly the same time, so their shared q/k rows are fetched once.
  int h, unit, half = 0;
  {
    int bid = blockIdx.x;
    if (MODE == kMap) {
      // the B halves (which walk the chunks) take the first half of the grid and
      // start at once; the A halves mostly stop after the decay scan
      const int hgrid = (int)(gridDim.x >> 1);
      half = bid < hgrid ? 1 : 0;  // 0: A columns, 1: B columns
      bid -= half ? 0 : hgrid;
    }
    const int r = Hv / Hk, rw = r / NH;
    const int x = bid & 7, y = bid >> 3;
    const int member = y % rw;
    const int pair = (y / rw) * 8 + x;  // (unit, q/k head) index
    h = (pair % Hk) * r + member * NH + hh;
    unit = pair / Hk;
  }
  const int gq = h / (Hv / Hk);
  const bool withV = MODE == kFull || half == 1;

  int segi;
  if (P.one_seq && one_seq_table_bad(P.cu, P.T)) return;
  const int nseg1 = P.one_seq ? seg_count(P.T, P.seg_len) : 0;  // one sequence: its segments
  if (MODE == kFull) {
    if (unit >= (P.one_seq ? nseg1 : P.hdr[0])) return;
    segi = P.one_seq ? unit : P.order[unit];
  } else {
    if (unit >= (P.one_seq ? nseg1 - 1 : P.hdr[1])) return;
    segi = P.one_seq ? unit : P.map_seg[unit];
  }
  const SegInfo seg = P.one_seq ? seg_record(0, 0, P.T, segi, P.seg_len, 0, 0) : P.segs[segi];
  const int seq_begin = seg.seq_begin;
  const int seg_end = seg.begin + seg.len;

  unsigned char *const hblk = smem + L::HEAD + hh * L::H_BYTES;  // this head's block
  bf16_t *const sQf = reinterpret_cast<bf16_t *>(smem + L::QF);  // fp16 bits
  bf16_t *const sKf = reinterpret_cast<bf16_t *>(smem + L::KF);  // fp16 bits
  bf16_t *const sKT = reinterpret_cast<bf16_t *>(smem + L::KT);  // fp16 bits
  float *const sConvW = reinterpret_cast<float *>(smem + L::CONVW);
  float *const sNW = reinterpret_cast<float *>(smem + L::NW);
  float *const sVT = reinterpret_cast<float *>(hblk + L::H_VT);
  // the o tile has a region of its own: a wave writes it while the head's other waves
  // may still read their V^T rows
  float *const sO = reinterpret_cast<float *>(hblk + L::H_O);
  float *const sGates = reinterpret_cast<float *>(hblk + L::H_GATES);
  float *const sMdiag = reinterpret_cast<float *>(hblk + L::H_MDIAG);
  bf16_t *const sLo = reinterpret_cast<bf16_t *>(hblk + L::H_LO);
  bf16_t *const sTd = reinterpret_cast<bf16_t *>(hblk + L::H_TD);
  bf16_t *const sM = reinterpret_cast<bf16_t *>(hblk + L::H_M);

  // ---- roles of the prologue ----------------------------------------------------
  // Before the first barrier every wave convolves q (roles 0-1) or k (roles 2-3):
  // TPT tokens x 8 channels per thread, the 16 lanes of a token row spanning its 128
  // channels (for the L2 norm); wave qi of its kind takes tokens 4 TPT qi .. + 4 TPT - 1.
  // Map mode needs no q: all four waves convolve k (and the A half needs no v).  After
  // the barrier every thread convolves 4 tokens x 4 channels of its head's v, which
  // only the right-hand side (after barrier 2) reads.
  constexpr int TPT = (NH == 2 || MODE == kMap) ? 2 : 4;  // q/k tokens per thread
  const int role = (MODE == kMap || wave >= 2) ? 1 : 0;   // uniform per wave
  int cg = lane & 15;                  // q/k channels 8cg .. 8cg+7
  // the wave's index among the waves of its kind (q or k), 16 / TPT tokens each
  const int qi = MODE == kMap ? wave : NH == 2 ? 2 * hh + (wave & 1) : (wave & 1);
  int tbase = TPT * (4 * qi + (lane >> 4));
  // v channels 4cv .. 4cv+3 of the head, ht = the thread's index among its head's 256;
  // cv rotates the 5 lane bits so that the 8 lanes of one 16-byte LDS write cycle take
  // cv values 4 apart: their V^T rows 4cv + cc lie in 8 different 16-row blocks, which
  // the tile's swizzle spreads over all banks
  const int ht = wave * 64 + lane;
  int cv = ((ht & 7) << 2) | ((ht >> 3) & 3);
  int vbase = (ht >> 5) * 4;           // v tokens vbase .. vbase+3
  // Re-derive the lane coordinates behind an optimisation barrier after every
  // workgroup barrier, so that LDS addresses are formed next to their use
  // instead of being hoisted out of the chunk loop (and spilled).  The v-conv
  // coordinates (cv, vbase) are left to the compiler: it keeps their addresses in
  // registers without spilling, which measured ~1 % faster.
  auto refresh = [&]() {
    tid = opaque(tid);
    roles();
    lane = tid & 63;
    ln = lane & 15;
    lg = lane >> 4;
    cg = opaque(cg);
    tbase = opaque(tbase);
  };
  const bool qk_on = MODE == kFull || role == 1;
  const bool v_on = withV;

  // conv taps -> LDS: q channels 0..127, k 128..255, then 128 per v head of the workgroup
  for (int i = tid; i < (256 + 128 * NH) * 4; i += kTh) {
    const int ch = i >> 2, tap = i & 3;
    int64_t c;
    if (ch < 128) c = (int64_t)gq * kD + ch;
    else if (ch < 256) c = (int64_t)Hk * kD + (int64_t)gq * kD + (ch - 128);
    else c = 2LL * Hk * kD + (int64_t)(h - hh) * kD + (ch - 256);
    sConvW[(ch >> 3) * kConvGS + (ch & 7) * 4 + tap] = P.conv_w[c * 4 + tap] * kConvScale;
  }

  // this wave's q or k columns and the head's v columns (uniform), token strides
  const T *src = (role == 0 ? (const T *)P.q : (const T *)P.k) + (int64_t)gq * kD;
  const T *vsrc = (const T *)P.v + (int64_t)h * kD;
  const int qk_stride = Hk * kD, v_stride = Hv * kD;
  const T *hist = nullptr, *vhist = nullptr;
  if (P.conv_in) {
    const T *hs = (const T *)P.conv_in + (int64_t)seg.seq * 3 * P.Cc;
    hist = hs + (int64_t)role * Hk * kD + (int64_t)gq * kD + cg * 8;
    vhist = hs + 2LL * Hk * kD + (int64_t)h * kD + cv * 4;
  }

  // raw rows for one chunk: rows base-3 .. base+TPT-1 (q/k), base-3 .. base+3 (v)
  // relative to the chunk start
  typedef RawN<T, 8> RQ;
  typedef RawN<T, 4> RV;
  constexpr int kQR = TPT + 3;
  uint32_t raw[kQR][RQ::W], vraw[7][RV::W];
  // Interior chunks use one buffer per stream (rows at or past the segment end
  // read as zero); chunks that start within 3 rows of the sequence start take
  // rows before it from the conv history (or zero them at use) and clamp rows
  // past the segment (masked at use).
  auto load_chunk = [&](int t0) {
    if (t0 - 3 >= seq_begin) {
      const int nrows = min(seg_end - (t0 - 3), kChunk + 3);
      if (qk_on) {
        const int rowb = qk_stride * (int)sizeof(T);
        const rsrc_t rs = buf(src + (int64_t)(t0 - 3) * qk_stride, nrows * rowb);
        const uint32_t lo = (uint32_t)(tbase * rowb + cg * 8 * (int)sizeof(T));
#pragma unroll
        for (int rr = 0; rr < kQR; ++rr) RQ::load_buf(raw[rr], rs, lo + rr * rowb);
      }
      if (v_on) {
        const int rowb = v_stride * (int)sizeof(T);
        const rsrc_t rs = buf(vsrc + (int64_t)(t0 - 3) * v_stride, nrows * rowb);
        const uint32_t lo = (uint32_t)(vbase * rowb + cv * 4 * (int)sizeof(T));
#pragma unroll
        for (int rr = 0; rr < 7; ++rr) RV::load_buf(vraw[rr], rs, lo + rr * rowb);
      }
    } else {
      if (qk_on) {
#pragma unroll
        for (int rr = 0; rr < kQR; ++rr) {
          const int tau = t0 + tbase - 3 + rr;
          const int tc = min(max(tau, seq_begin), seg_end - 1);
          RQ::load(raw[rr], (tau < seq_begin && hist) ? hist + (3 + tau - seq_begin) * P.Cc
                                                      : src + (int64_t)tc * qk_stride + cg * 8);
        }
      }
      if (v_on) {
#pragma unroll
        for (int rr = 0; rr < 7; ++rr) {
          const int tau = t0 + vbase - 3 + rr;
          const int tc = min(max(tau, seq_begin), seg_end - 1);
          RV::load(vraw[rr], (tau < seq_begin && vhist) ? vhist + (3 + tau - seq_begin) * P.Cc
                                                        : vsrc + (int64_t)tc * v_stride + cv * 4);
        }
      }
    }
  };

  // ---- state accumulators ---------------------------------------------------------
  // Hacc[dt][ct]: rows (dk) 16dt + 4lg + i, column (dv) 32*wave + 16ct + ln.
  f32x4 Hacc[8][2];
  {
    const float *H0 = nullptr;
    if (MODE == kFull) {
      if (seg.idx > 0) {
        // start state after the previous segment: its B map itself when that
        // segment's A map is zero, else what the combine pass wrote
        const int64_t m = P.one_seq ? segi - 1 : P.segs[segi - 1].map;
        H0 = P.map_zero[m * Hv + h] ? P.maps + ((m * Hv + h) * 2 + 1) * kD * kD
                                    : P.starts + ((int64_t)segi * Hv + h) * kD * kD;
      } else if (P.init_state) {
        // A sequence of several segments starts from the copy of its initial state that
        // the combine pass made: its last segment writes final_state in this launch,
        // and final_state may alias init_state.
        H0 = seg.nseg > 1 ? P.starts + ((int64_t)segi * Hv + h) * kD * kD
                          : P.init_state + ((int64_t)seg.seq * Hv + h) * kD * kD;
      }
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * dt + 4 * lg + i, col = 32 * wave + 16 * ct + ln;
          float x = 0.f;
          if (MODE == kFull) x = H0 ? H0[row * kD + col] : 0.f;
          else if (half == 0) x = row == col ? 1.f : 0.f;
          Hacc[dt][ct][i] = x;
        }
  }
  // The accumulators hold sigma H with sigma = 2^sexp, a power of two per wave, and
  // hb bounds |sigma H| (both uniform).  The start puts max |H0| in [2^13, 2^14).
  int sexp = 0;
  float hb = 0.f;
  {
    float m = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(Hacc[dt][ct][i]));
    m = wave_max_nonneg(m);
    const int eb = exp_bits(m);
    if (eb > 0 && eb < 255) sexp = min(max(140 - eb, -60), 60);
    const float s0 = pow2f(sexp);
    hb = m * s0;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) Hacc[dt][ct][i] *= s0;
  }

  const float A_log_h = P.A_log[h], dt_bias_h = P.dt_bias[h];
  // Gates of one chunk, computed by wave 3 one chunk ahead (where it has slack):
  // inputs of token `lane` of the chunk starting at t0g, then the gate vectors of
  // its nv tokens (tokens past nv get g = 0, beta = 0) into buffer gbuf.
  auto load_gates = [&](int t0g, float &ga, float &gb) {
    const int tc = min(t0g + lane, seg_end - 1);
    ga = P.a[(int64_t)tc * Hv + h];
    gb = P.b[(int64_t)tc * Hv + h];
  };
  auto write_gates = [&](float *gbuf, int nv, float ga, float gb) {
    float g = 0.f, be = 0.f;
    if (lane < nv) {
      g = log_decay_fast(ga, A_log_h, dt_bias_h);
      be = sigmoid_fast(gb);
    }
    g = wave_inclusive_sum(g);  // G: inclusive cumsum of g
    const float GC = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g), 63));
    if (lane < kChunk) {
      const float gam = __expf(g);
      gbuf[GB_BETA * kChunk + lane] = be;
      gbuf[GB_G * kChunk + lane] = g;
      gbuf[GB_GAM * kChunk + lane] = gam;
      gbuf[GB_BG * kChunk + lane] = be * gam;
      gbuf[GB_DEC * kChunk + lane] = __expf(GC - g);
      gbuf[GB_BV * kChunk + lane] = be * (1.0f / kConvScale);
    }
  };
  if (MODE == kFull && tid < kD) sNW[tid] = P.norm_w ? P.norm_w[tid] : 1.0f;
  const int nchunks = (seg.len + kChunk - 1) / kChunk;
  const bool last_seg = seg.idx == seg.nseg - 1;

  // Map mode: skip work whose contribution is provably below fp32 resolution.
  // Each token multiplies the state by alpha_t (I - beta_t k_t k_t^T), whose
  // 2-norm is <= alpha_t (beta in [0,1], |k| <= 1), so everything before chunk c
  // reaches the segment end scaled by at most e^{S_c}, S_c = sum of g over
  // chunks c.. of the segment.  With S_c <= -100 ln 2 that part is dropped: the
  // B map starts at the last such chunk, and the A map is zero if S_0 is.
  int c_begin = 0;
  if (MODE == kMap) {
    // Chunk sums of g from the segment end, four chunks (one per wave) at a time,
    // until the suffix sum S reaches the threshold.  g <= 0, so the first chunk
    // where it does is the truncation point of the B map, and then the whole
    // segment's sum is below the threshold too: the A map is zero.  Only if no
    // suffix reaches it does the scan cover every chunk (A and B need them all).
    float *sChG = sVT;  // V^T is not in use before the chunk loop
    const float thr = -69.31471805599453f;  // ln 2^-100
    float S = 0.f;
    bool reached = false;
    for (int top = nchunks - 1; top >= 0 && !reached; top -= kWaves) {
      const int cc = top - wave;
      if (cc >= 0) {  // chunk sum, fixed order
        const int tau = seg.begin + cc * kChunk + lane;
        float g = (lane < kChunk && tau < seg_end)
                      ? log_decay(P.a[(int64_t)tau * Hv + h], A_log_h, dt_bias_h) : 0.f;
        g = wave_sum(g);
        if (lane == 0) sChG[cc] = g;
      }
      __syncthreads();
      for (int k = 0; k < kWaves && top - k >= 0; ++k) {  // every thread, same order
        S += sChG[top - k];
        if (S <= thr) {
          c_begin = top - k;
          reached = true;
          break;
        }
      }
      __syncthreads();  // sChG reuse by the next batch
    }
    if (half == 0) {
      // A map zero to fp32 resolution: flag it instead of storing it
      if (tid == 0) P.map_zero[(int64_t)unit * Hv + h] = reached ? 1 : 0;
      if (reached) return;
      c_begin = 0;  // otherwise the A map needs every chunk
    }
  }
  if (nchunks > 0) load_chunk(seg.begin + c_begin * kChunk);
  if (wave == 3 && c_begin < nchunks) {  // the first chunk's gates
    float ga, gb;
    load_gates(seg.begin + c_begin * kChunk, ga, gb);
    write_gates(sGates + (c_begin & 1) * kGateN, min(kChunk, seg_end - seg.begin - c_begin * kChunk),
                ga, gb);
  }
  __syncthreads();  // conv weights, first gates

  for (int c = c_begin; c < nchunks; ++c) {
    refresh();
    const int t0 = seg.begin + c * kChunk;
    const int nvalid = min(kChunk, seg_end - t0);

    // this chunk's gate vectors (written one chunk ahead)
    const float *const gcur = sGates + (c & 1) * kGateN;
    const float *const sBeta = gcur + GB_BETA * kChunk, *const sG = gcur + GB_G * kChunk;
    const float *const sGam = gcur + GB_GAM * kChunk, *const sBG = gcur + GB_BG * kChunk;
    const float *const sDec = gcur + GB_DEC * kChunk, *const sBv = gcur + GB_BV * kChunk;
    // gC = gamma_C, the chunk's decay (the same in every lane)
    const float gC = sGam[kChunk - 1];
    // the next chunk's gate inputs (wave 3), issued first and consumed in the gram
    // phase under the same condition (left undefined otherwise, so that no select
    // waits for the loads here)
    float ga, gb;
    const bool gates_next = wave == 3 && c + 1 < nchunks;
    if (gates_next) load_gates(t0 + kChunk, ga, gb);

    // ================= prologue: conv + SiLU (+ L2) -> LDS ========================
    // Issue priority follows each phase's longest waves: here the k waves (K^T
    // regrouping), from barrier 1 to barrier 2 roles 0 and 1 (their diagonal gram
    // tiles, L/M, the 16x16 inverses, then the q waves' prefetch), and after that
    // the second head's waves (NH = 2), which the SIMDs otherwise serve after the older
    // first-head waves, so that they do not arrive last at barrier 1.  With NH = 1 the
    // two workgroups on a compute unit fill the SIMDs between these phases.
    __builtin_amdgcn_s_setprio(0);
    if (MODE == kFull && wave >= 2) __builtin_amdgcn_s_setprio(1);
    if (t0 - 3 < seq_begin && !hist) {  // rows before the sequence read as zero
#pragma unroll
      for (int rr = 0; rr < kQR; ++rr)
        if (t0 + tbase - 3 + rr < seq_begin)
#pragma unroll
          for (int w = 0; w < RQ::W; ++w) raw[rr][w] = 0u;
#pragma unroll
      for (int rr = 0; rr < 7; ++rr)
        if (t0 + vbase - 3 + rr < seq_begin)
#pragma unroll
          for (int w = 0; w < RV::W; ++w) vraw[rr][w] = 0u;
    }
    if (qk_on) {  // q or k: TPT tokens x 8 channels, L2 over the head's 128 channels
      float x[TPT][8];
      conv_silu_rows<T, TPT, 8>(raw, sConvW + (role * 16 + cg) * kConvGS, x);
      // x = kConvScale SiLU(u): dividing by the norm of x takes out |kConvScale|,
      // the sign is applied here and eps scales with kConvScale^2.  q and k stay
      // unit-norm (q_scale multiplies the products that use q instead), so their
      // fp16 copies cannot overflow.
      const float scale0 = -1.0f;
      const float eps = P.l2_eps * (kConvScale * kConvScale);
#pragma unroll
      for (int r = 0; r < TPT; ++r) {
        float ss = 0.f;
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) ss += x[r][cc] * x[r][cc];
        ss = row16_sum(ss);
        const float f = scale0 * rsq_normal(ss + eps);
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) x[r][cc] *= f;
      }
      // fp16 rows of q (the gram products and Q H) or k (the gram products), and the
      // fp16 k rows regrouped into K^T (right-hand side and state update)
      uint32_t fw[TPT][4];  // token r: fp16 channels (2e, 2e+1) in word e
#pragma unroll
      for (int r = 0; r < TPT; ++r) {
#pragma unroll
        for (int e = 0; e < 4; ++e) fw[r][e] = pk_f16(x[r][2 * e], x[r][2 * e + 1]);
        *reinterpret_cast<uint4 *>((role == 0 ? sQf : sKf) + (tbase + r) * kRowS + cg * 8) =
            make_uint4(fw[r][0], fw[r][1], fw[r][2], fw[r][3]);
      }
      if (role == 1) {
        // K^T [dk][tok]: fp16 k regrouped by channel, 2 bytes per token; rows 8cg + cc
        // (cc < 8) share row >> 4 = cg >> 1.  Tokens (2p, 2p+1) of channel cc are half
        // (cc & 1) of word cc/2 of tokens 2p, 2p+1.  The 4-token group tbase >> 2 is
        // swizzled; TPT = 2 fills half of it (4 bytes), TPT = 4 all of it (8 bytes).
        const int swz = ((((tbase >> 2) ^ (cg >> 1)) & 7) << 2) + (tbase & 2);
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) {
          const uint32_t sel = (cc & 1) ? 0x07060302u : 0x05040100u;
          const int e = cc >> 1;
          bf16_t *const dst = sKT + (cg * 8 + cc) * kTokS + swz;
          if constexpr (TPT == 4)
            *reinterpret_cast<uint2 *>(dst) = make_uint2(__builtin_amdgcn_perm(fw[1][e], fw[0][e], sel),
                                                         __builtin_amdgcn_perm(fw[3][e], fw[2][e], sel));
          else
            *reinterpret_cast<uint32_t *>(dst) = __builtin_amdgcn_perm(fw[1][e], fw[0][e], sel);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();  // (1) prologue tiles ready
    refresh();
    if (MODE == kFull && wave < 2) __builtin_amdgcn_s_setprio(1);

    if (v_on) {  // v: 4 tokens x 4 channels -> fp32 V^T [dv][tok], 16 bytes per channel
      float x[4][4];
      conv_silu_rows<T, 4, 4>(vraw, sConvW + (32 + 16 * hh + (cv >> 1)) * kConvGS + (cv & 1) * 16,
                              x);
      // rows 4cv + cc share row >> 4 = cv >> 2; vbase = 4 * (4-token group)
      const int swz = ((vbase >> 2) ^ ((cv >> 2) & 7)) << 2;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc)
        *reinterpret_cast<f32x4 *>(sVT + (cv * 4 + cc) * kVtS + swz) =
            f32x4{x[0][cc], x[1][cc], x[2][cc], x[3][cc]};
    }

    // this chunk's gate z (raw bits, consumed by the epilogue) and the next chunk's
    // raw rows (consumed by the next prologue) stay in flight during the math; z is
    // issued first so that waiting for it never waits for the prefetch
    // epilogue layout: token ht >> 3, columns 8e..8e+7 and 64+8e..64+8e+7 with
    // e = ht & 7 (two 16-byte bf16 blocks per thread for z and o)
    typedef RawN<T, 8> RZ;
    uint32_t zw[2][RZ::W];
    if (MODE == kFull) {
      // one buffer over this chunk's rows (uniform); tokens at or past nvalid read as zero
      const int rowb = Hv * kD * (int)sizeof(T);
      const rsrc_t zs = buf((const T *)P.z + ((int64_t)t0 * Hv + h) * kD, nvalid * rowb);
      const int zt = wave * 64 + lane;
      const uint32_t zo = (uint32_t)((zt >> 3) * rowb + 8 * (zt & 7) * (int)sizeof(T));
      RZ::load_buf(zw[0], zs, zo);
      RZ::load_buf(zw[1], zs, zo + 64 * (int)sizeof(T));
    }

    // ================= gram products K K^T (and Q K^T) =========================
    // lower 16x16 tiles of the 32x32 products: wave 0 (0,0), wave 1 (1,1), wave 2
    // (1,0); the diagonal-tile waves also form that block's (I + L)^-1
    const bool gram_on = wave < 3;
    const int ti = wave == 0 ? 0 : 1, tj = wave == 1 ? 1 : 0;
    f32x4 kk = {0.f, 0.f, 0.f, 0.f}, qk = {0.f, 0.f, 0.f, 0.f};
    if (gram_on) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int col = 32 * kb + 8 * lg;
        const u16x8 bk = *reinterpret_cast<const u16x8 *>(sKf + (16 * tj + ln) * kRowS + col);
        const u16x8 ak = *reinterpret_cast<const u16x8 *>(sKf + (16 * ti + ln) * kRowS + col);
        kk = mfma16h(ak, bk, kk);
        if (MODE == kFull) {
          const u16x8 aq = *reinterpret_cast<const u16x8 *>(sQf + (16 * ti + ln) * kRowS + col);
          qk = mfma16h(aq, bk, qk);
        }
      }
    }
    // L, M tiles to LDS; the diagonal-tile waves form (I + L_bb)^-1 - I.  The gates
    // were written a chunk ahead, -L, T_bb - I and M have regions of their own: no
    // barrier after the gram products
    if (gram_on) {
      const int cj = 16 * tj + ln;
      const float Gj = sG[cj];
      const f32x4 Gr = *reinterpret_cast<const f32x4 *>(sG + 16 * ti + 4 * lg);
      const f32x4 Br = *reinterpret_cast<const f32x4 *>(sBeta + 16 * ti + 4 * lg);
      float l[4], d[4];  // L and the decay e^{G_i - G_j} (j < i; 0 and 1 elsewhere)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool low = cj < 16 * ti + 4 * lg + i;
        d[i] = __expf(low ? Gr[i] - Gj : 0.f);
        l[i] = low ? Br[i] * d[i] * kk[i] : 0.f;
      }
      if (MODE == kFull) {  // M with zero diagonal and upper part
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool low = cj < 16 * ti + 4 * lg + i;
          sM[(16 * ti + 4 * lg + i) * kSqS + cj] = f2h(low ? d[i] * qk[i] : 0.f);
        }
      }
      if (ti != tj) {  // wave 2: the off-diagonal block of -L
#pragma unroll
        for (int i = 0; i < 4; ++i) sLo[(16 * ti + 4 * lg + i) * kSqS + cj] = f2h(-l[i]);
      } else {
        // diagonal block: M's diagonal (fp32) and (I + L_bb)^-1 - I from the C-layout
        // tiles of -L^T (mc) and -L (mt)
        if (MODE == kFull) {
          const int di = ln - 4 * lg;  // the lane's diagonal element, if any
          if (di >= 0 && di < 4) {
            const float qd = di == 0 ? qk[0] : (di == 1 ? qk[1] : (di == 2 ? qk[2] : qk[3]));
            sMdiag[cj] = qd;
          }
        }
        const float Bj = sBeta[cj];
        f32x4 mc, mt;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool up = 16 * ti + 4 * lg + i < cj;
          const float du = __expf(up ? Gj - Gr[i] : 0.f);
          mt[i] = -l[i];
          mc[i] = up ? -(Bj * du * kk[i]) : 0.f;
        }
        const f32x4 tt = unit_lower_inverse_t(mc, mt, ln, lg);  // row ln of T, cols 4lg..
        float e[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) e[i] = tt[i] - (4 * lg + i == ln ? 1.0f : 0.0f);
        *reinterpret_cast<uint2 *>(sTd + (16 * ti + ln) * kTdS + 4 * lg) =
            make_uint2(pk_f16(e[0], e[1]), pk_f16(e[2], e[3]));
      }
    }
    if (MODE == kFull && wave == 3) {  // zero the upper tile (0,1) of M read by M U
#pragma unroll
      for (int i = 0; i < 4; ++i) sM[(4 * lg + i) * kSqS + 16 + ln] = 0;
    }
    // the next chunk's gates (wave 3, which has no diagonal tile)
    if (gates_next)
      write_gates(sGates + ((c + 1) & 1) * kGateN, min(kChunk, seg_end - t0 - kChunk), ga, gb);
    // next chunk's raw rows: the k waves (off the diagonal tiles) go first so that
    // the q waves' loads after the barrier do not queue behind theirs
    if (role == 1 && c + 1 < nchunks) load_chunk(t0 + kChunk);
    __syncthreads();  // (2) -L, M, T_bb - I, V^T and the next gates ready
    refresh();
    if (role == 0 && c + 1 < nchunks) load_chunk(t0 + kChunk);  // next chunk's raw rows

    __builtin_amdgcn_s_setprio(0);
    if (NH == 2 && hh == 1) __builtin_amdgcn_s_setprio(1);

    // ================= K H and Q H, U by one triangular solve, O, H update ==========
    // With W = T diag(beta gamma) K and Utilde = T diag(beta) V, the new values are
    //   U = Utilde - W H = T (diag(beta) V - diag(beta gamma) K H),
    // so the chunk needs K H (the same products as W H) and one solve of this wave's
    // 32 columns, with no W tile shared between the waves.
    // The accumulators hold sigma H (sigma = 2^sexp per wave) with |sigma H| below 2^14
    // (hb bounds it, see the update), so H enters K H and Q H as fp16 B operands:
    // Hb[kb][ct] slots 8lg+j <-> dk 32kb + 4lg + j (j<4), 32kb + 16 + 4lg + j - 4 (j >= 4).
    // K and Q are unit-norm.
    f32x4 Uacc[2][2], Oacc[2][2];  // [row tile of 16 tokens][column tile]
    {
      u16x8 Hb[4][2];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) Hb[kb][ct] = pack_h(Hacc[2 * kb][ct], Hacc[2 * kb + 1][ct]);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          Uacc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
          Oacc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      // k-block outer: four independent accumulators per product and block
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          const u16x8 ak = load_a_perm(sKf + (16 * rt + ln) * kRowS, 32 * kb, 32 * kb + 16, lg);
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) Uacc[rt][ct] = mfma16h(ak, Hb[kb][ct], Uacc[rt][ct]);
          if (MODE == kFull) {
            const u16x8 aq = load_a_perm(sQf + (16 * rt + ln) * kRowS, 32 * kb, 32 * kb + 16, lg);
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) Oacc[rt][ct] = mfma16h(aq, Hb[kb][ct], Oacc[rt][ct]);
          }
        }
      }
    }
    // Right-hand side R = sigma beta V - beta gamma (K sigma H) in fp32 (the beta vector of
    // V also holds 1 / kConvScale), then scaled by s = 2^rexp, which puts the wave's
    // largest |R| in [2^3, 2^4): the solution X = s sigma U is then at most 32 times
    // that, and the intermediate rows of the blocked substitution at most 17 times
    // more, all inside fp16's range.
    int rexp = 0;
    {
      const float sg = pow2f(sexp);
      float mr = 0.f;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const f32x4 be = *reinterpret_cast<const f32x4 *>(sBv + 16 * rt + 4 * lg);
        const f32x4 bg = *reinterpret_cast<const f32x4 *>(sBG + 16 * rt + 4 * lg);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          f32x4 vv = {0.f, 0.f, 0.f, 0.f};
          if (withV) {
            const int dcol = 32 * wave + 16 * ct + ln;
            vv = *reinterpret_cast<const f32x4 *>(sVT + tok_swz(dcol, 16 * rt + 4 * lg, kVtS));
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            Uacc[rt][ct][i] = fmaf(-bg[i], Uacc[rt][ct][i], (be[i] * sg) * vv[i]);
            mr = fmaxf(mr, fabsf(Uacc[rt][ct][i]));
          }
        }
      }
      const int eb = exp_bits(wave_max_nonneg(mr));
      if (eb > 0 && eb < 255) rexp = min(max(130 - eb, -120), 120);
      const float sr = pow2f(rexp);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i) Uacc[rt][ct][i] *= sr;
    }
    // block forward substitution (I + L) X = R over two row blocks of 16 tokens:
    //   X_0 = (I + (T_00 - I)) R_0,   X_1 = (I + (T_11 - I)) (R_1 - L_10 X_0)
    // on 16 x 16 blocks (K = 16): the A operand is row ln of the block, columns
    // 4lg..4lg+3, the B operand the C-layout tile itself; the identity part in fp32
    {
      const f16x4_t at0 = *reinterpret_cast<const f16x4_t *>(sTd + ln * kTdS + 4 * lg);
      f16x4_t x0h[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        Uacc[0][ct] = mm16(at0, h4(Uacc[0][ct]), Uacc[0][ct]);
        x0h[ct] = h4(Uacc[0][ct]);
      }
      const f16x4_t a10 = *reinterpret_cast<const f16x4_t *>(sLo + (16 + ln) * kSqS + 4 * lg);  // -L_10
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) Uacc[1][ct] = mm16(a10, x0h[ct], Uacc[1][ct]);
      const f16x4_t at1 = *reinterpret_cast<const f16x4_t *>(sTd + (16 + ln) * kTdS + 4 * lg);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) Uacc[1][ct] = mm16(at1, h4(Uacc[1][ct]), Uacc[1][ct]);
    }
    // The chunk's scale step rho (a power of two): the new state rho (gamma_C sigma H +
    // K^T sigma u) and the fp16 operands rho sigma U stay below 2^14 with the bound
    // hb' = gamma_C hb + 32 max|sigma U| (|K^T u| <= 32 max|u| for unit keys, u = U
    // e^{G_C - G}, |u| <= |U|) placed in [2^13, 2^14); hb tracks a bound on |sigma H|.
    // sigma stays within 2^-60 .. 2^60; rho = 1 when the bound is zero or not finite.
    // Uacc holds X = s sigma U; f = rho / s brings it to rho sigma U.
    float rho, f;
    {
      float mx = 0.f;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(Uacc[rt][ct][i]));
      const float mu = wave_max_nonneg(mx) * pow2f(-rexp);
      const float bound = fmaf(32.0f, mu, gC * hb);
      const int eb = exp_bits(bound);
      int snew = sexp;
      if (eb > 0 && eb < 255) snew = min(max(sexp + 140 - eb, -60), 60);
      rho = pow2f(snew - sexp);
      // below 2^-126 the U terms are far under fp32 resolution of the state
      f = pow2f(min(max(snew - sexp - rexp, -126), 127));
      hb = bound * rho;
      sexp = snew;
    }
    // X -> rho sigma U, which every consumer below takes as it is (f is a power of two)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) Uacc[rt][ct][i] *= f;
    if (MODE == kFull) {  // O = gamma Q H + diag(M) U + M_off U, scaled by rho sigma / q_scale
      u16x8 Ub[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) Ub[ct] = pack_h(Uacc[0][ct], Uacc[1][ct]);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        // rho is a power of two: folding it into the row factor changes no rounding
        f32x4 gm = *reinterpret_cast<const f32x4 *>(sGam + 16 * rt + 4 * lg);
        const f32x4 md = *reinterpret_cast<const f32x4 *>(sMdiag + 16 * rt + 4 * lg);
#pragma unroll
        for (int i = 0; i < 4; ++i) gm[i] *= rho;
        const u16x8 am = load_a_perm(sM + (16 * rt + ln) * kSqS, 0, 16, lg);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            Oacc[rt][ct][i] = fmaf(md[i], Uacc[rt][ct][i], Oacc[rt][ct][i] * gm[i]);
          Oacc[rt][ct] = mfma16h(am, Ub[ct], Oacc[rt][ct]);
        }
      }
    }
    // state update H = gamma_C H + K^T diag(e^{G_C - G}) U, one fp16 pass (K unit-norm)
    {
      uint32_t uh[2][4];  // [ct]: tokens 4lg.. of row tile 0, then of row tile 1
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const f32x4 dec = *reinterpret_cast<const f32x4 *>(sDec + 16 * rt + 4 * lg);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          uh[ct][2 * rt] = pk_f16(Uacc[rt][ct][0] * dec[0], Uacc[rt][ct][1] * dec[1]);
          uh[ct][2 * rt + 1] = pk_f16(Uacc[rt][ct][2] * dec[2], Uacc[rt][ct][3] * dec[3]);
        }
      }
      u16x8 Uh[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        Uh[ct] = __builtin_bit_cast(u16x8, make_uint4(uh[ct][0], uh[ct][1], uh[ct][2], uh[ct][3]));
      const TokLane tl(ln, lg);
      const float gCr = gC * rho;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i) Hacc[dt][ct][i] *= gCr;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const u16x8 ak = load_a_tok(sKT, tl, dt);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) Hacc[dt][ct] = mfma16h(ak, Uh[ct], Hacc[dt][ct]);
      }
    }

    // ================= epilogue: RMSNorm over 128 columns, SiLU(z) gate ============
    if (MODE == kFull) {  // this wave's 32 columns of o -> the fp32 o tile
      const float rsig = P.q_scale * pow2f(-sexp);  // O was scaled by sigma (new) / q_scale
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sO[(16 * rt + 4 * lg + i) * kOS + 32 * wave + 16 * ct + ln] = Oacc[rt][ct][i] * rsig;
    }
    __syncthreads();  // (3) o tile ready; this chunk's other LDS tiles are consumed
    refresh();
    if (MODE == kFull) {
      // token ht >> 3 (8 lanes per token), columns 8e.. and 64+8e.. with e = ht & 7;
      // the four 16-byte reads of a row are bank-conflict free with kOS = 132
      const int et = wave * 64 + lane;
      const int etok = et >> 3, e8 = 8 * (et & 7);
      const float *orow = sO + etok * kOS;
      float ov[16], nw[16];
      {
        const f32x4 r0 = *reinterpret_cast<const f32x4 *>(orow + e8);
        const f32x4 r2 = *reinterpret_cast<const f32x4 *>(orow + 64 + e8);
        const f32x4 r1 = *reinterpret_cast<const f32x4 *>(orow + e8 + 4);
        const f32x4 r3 = *reinterpret_cast<const f32x4 *>(orow + 68 + e8);
        const f32x4 w0 = *reinterpret_cast<const f32x4 *>(sNW + e8);
        const f32x4 w1 = *reinterpret_cast<const f32x4 *>(sNW + e8 + 4);
        const f32x4 w2 = *reinterpret_cast<const f32x4 *>(sNW + 64 + e8);
        const f32x4 w3 = *reinterpret_cast<const f32x4 *>(sNW + 68 + e8);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          ov[j] = r0[j]; ov[4 + j] = r1[j]; ov[8 + j] = r2[j]; ov[12 + j] = r3[j];
          nw[j] = w0[j]; nw[4 + j] = w1[j]; nw[8 + j] = w2[j]; nw[12 + j] = w3[j];
        }
      }
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) ss += ov[j] * ov[j];
      // sum over the 8 lanes of the token: quad butterflies, then the other quad
      ss += dpp_f<0xB1>(ss);  // quad_perm 1,0,3,2
      ss += dpp_f<0x4E>(ss);  // quad_perm 2,3,0,1
      ss += dpp_f<0x141>(ss);  // row_half_mirror
      // o * rsqrt(ms) * w * z * sigmoid(z) with the RMS folded into the sigmoid's
      // denominator: 1 / (sd (1 + e^-z)), sd = sqrt(ms + eps)
      const float ms = ss * (1.0f / kD) + P.rms_eps;
      const float sd = ms * rsq_normal(ms);
      float val[16], zv[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        zv[j] = RZ::get(zw[j >> 3], j & 7);
        const float e = __expf(-zv[j]);
        val[j] = ov[j] * nw[j] * __builtin_amdgcn_rcpf(fmaf(e, sd, sd));
      }
      if (P.gate == 0) {  // SiLU gate z sigmoid(z); the sigmoid gate stops at sigmoid(z)
#pragma unroll
        for (int j = 0; j < 16; ++j) val[j] *= zv[j];
      }
      // one buffer over this chunk's o rows: stores of tokens at or past nvalid are dropped
      const int rowb = Hv * kD * (int)sizeof(T);
      const rsrc_t os = buf((T *)P.o + ((int64_t)t0 * Hv + h) * kD, nvalid * rowb);
      const uint32_t oo = (uint32_t)(etok * rowb + e8 * (int)sizeof(T));
      OutRow<T>::store(os, oo, val);
      OutRow<T>::store(os, oo + 64 * (int)sizeof(T), val + 8);
    }
  }

  // ---- state out ---------------------------------------------------------------------
  float *Hout = nullptr;
  if (MODE == kFull) {
    if (last_seg) Hout = P.final_state + ((int64_t)seg.seq * Hv + h) * kD * kD;
  } else {
    Hout = P.maps + (((int64_t)unit * Hv + h) * 2 + half) * kD * kD;
  }
  if (Hout) {
    const float rsig = pow2f(-sexp);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          Hout[(16 * dt + 4 * lg + i) * kD + 32 * wave + 16 * ct + ln] = Hacc[dt][ct][i] * rsig;
  }
}

// ------------------------------------------------------------ segment table

// One workgroup: sequence lengths -> segments (prefix sums over sequences).
// cu_seqlens must have cu[0] = 0, cu[i] <= cu[i+1] and cu[N] = T; otherwise the
// table is left empty (no segment runs, o and the final states are not written)
// and g_prefill_bad_cu is set.
__global__ void __launch_bounds__(1024) segment_table_kernel(
    const int32_t *cu, int N, int64_t T, int seg_len, int64_t max_segments, int64_t max_maps,
    SegInfo *segs, int32_t *hdr, int32_t *map_seg, int32_t *seq_first, int32_t *order) {
  __shared__ int s_nseg[1024], s_nmap[1024];
  __shared__ int s_base_seg, s_base_map, s_bad;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_base_seg = 0;
    s_base_map = 0;
    s_bad = 0;
  }
  __syncthreads();
  if (cu) {  // validate the whole table first
    for (int n = tid; n < N; n += 1024) {
      const int b0 = cu[n], e0 = cu[n + 1];
      if (e0 < b0 || (n == 0 && b0 != 0) || (n == N - 1 && (int64_t)e0 != T)) s_bad = 1;
    }
    __syncthreads();
    if (s_bad) {
      if (tid == 0) {
        hdr[0] = 0;
        hdr[1] = 0;
        g_prefill_bad_cu = 1;
      }
      return;
    }
  }
  for (int n0 = 0; n0 < N; n0 += 1024) {
    const int n = n0 + tid;
    int b = 0, e = 0, ns = 0, nm = 0;
    if (n < N) {
      b = cu ? cu[n] : 0;
      e = cu ? cu[n + 1] : (int)T;
      b = max(0, min(b, (int)T));       // keep every access inside [0, T)
      e = max(b, min(e, (int)T));
      ns = seg_count(e - b, seg_len);
      nm = ns - 1;
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
      seq_first[n] = first;
      for (int s = 0; s < ns; ++s) {
        const int idx = first + s;
        if (idx >= max_segments) break;
        SegInfo si = seg_record(n, b, e, s, seg_len, first, firstmap);
        if (firstmap + s >= max_maps) si.map = -1;
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
  // The full pass's order: segments by chunk count, longest first, so that the shortest
  // ones run last and the final round of workgroups leaves little idle time (packed
  // sequences of different lengths).  A counting sort over the <= 256 + 1 chunk counts;
  // the order inside a count is whatever the atomics give, which changes no result
  // (every segment is computed the same way by whichever workgroup takes it).
  const int nseg_all = (int)min((int64_t)s_base_seg, max_segments);
  if (N == 1) {  // one sequence: equal segments, in order
    for (int i = tid; i < nseg_all; i += 1024) order[i] = i;
  } else {
    __threadfence_block();
    __syncthreads();  // the segment records are written
    constexpr int kBins = kMaxSegChunks + 1;
    static_assert(kBins <= 512, "bins of the order scan");
    // bin j (j < 512) counts the segments of kMaxSegChunks - j chunks (longest first)
    int *cnt = s_nseg;  // reused
    if (tid < 512) cnt[tid] = 0;
    __syncthreads();
    for (int i = tid; i < nseg_all; i += 1024)
      atomicAdd(&cnt[kMaxSegChunks - min((segs[i].len + kChunk - 1) / kChunk, kMaxSegChunks)], 1);
    __syncthreads();
    int *scan = s_nmap;  // exclusive prefix sums of the bins
    const int own = tid < 512 ? cnt[tid] : 0;
    if (tid < 512) scan[tid] = own;
    __syncthreads();
    for (int o = 1; o < 512; o <<= 1) {
      const int add = (tid < 512 && tid >= o) ? scan[tid - o] : 0;
      __syncthreads();
      if (tid < 512) scan[tid] += add;
      __syncthreads();
    }
    if (tid < 512) cnt[tid] = scan[tid] - own;
    __syncthreads();
    for (int i = tid; i < nseg_all; i += 1024)
      order[atomicAdd(&cnt[kMaxSegChunks - min((segs[i].len + kChunk - 1) / kChunk, kMaxSegChunks)], 1)] = i;
  }
  if (tid == 0) {
    // (cannot happen for a valid table; kept so that no segment index ever passes
    // the workspace tables)
    const bool ok = s_base_seg <= max_segments && s_base_map <= max_maps;
    hdr[0] = ok ? s_base_seg : 0;
    hdr[1] = ok ? s_base_map : 0;
    if (!ok) g_prefill_bad_cu = 1;
  }
}

// Host side: read and clear the current device's invalid-cu_seqlens flag
// (synchronous; the caller has synchronised the stream that ran the prefill).
hipError_t take_prefill_error(int *flag) {
  int v = 0;
  hipError_t e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_prefill_bad_cu), sizeof(int), 0,
                                     hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  *flag = v;
  if (v) {
    const int zero = 0;
    e = hipMemcpyToSymbol(HIP_SYMBOL(g_prefill_bad_cu), &zero, sizeof(int), 0,
                          hipMemcpyHostToDevice);
  }
  return e;
}

// ------------------------------------------------------------ combine (pass 2)
// Per (sequence, v head, 16-column slice): H_0 = init; H_{s+1} = A_s H_s + B_s.
// Where A_s is zero (flagged by the map pass) H_{s+1} = B_s, which the full pass
// reads from the map itself; only the start states after a non-zero A map are
// computed and written here.
__global__ void __launch_bounds__(256) combine_kernel(const SegInfo *segs, const int32_t *hdr,
                                                      const int32_t *seq_first, int N,
                                                      const float *init_state, const float *maps,
                                                      const int32_t *map_zero, float *starts,
                                                      int Hv, int one_seq, int seg_len, int T,
                                                      const int32_t *cu) {
  __shared__ float sH[kD][17];
  const int slice = blockIdx.x % 8;
  const int h = (blockIdx.x / 8) % Hv;
  const int n = blockIdx.x / (8 * Hv);  // sequence
  if (n >= N) return;
  // its first segment (one sequence without a table: segment 0, records formed here)
  if (one_seq && one_seq_table_bad(cu, T)) return;
  const int segi = one_seq ? 0 : seq_first[n];
  if (!one_seq && (segi < 0 || segi >= hdr[0])) return;  // (no segments: invalid table)
  const SegInfo s0 = one_seq ? seg_record(0, 0, T, 0, seg_len, 0, 0) : segs[segi];
  if (s0.nseg < 2) return;
  const int tid = threadIdx.x;
  const int row = tid >> 1, c0 = (tid & 1) * 8;  // 8 outputs per thread
  const int col0 = slice * 16 + c0;
  float hreg[8];
  // H_s lives in hreg once loaded (have), else it is src (NULL: zeros)
  const float *src = init_state ? init_state + ((int64_t)s0.seq * Hv + h) * kD * kD : nullptr;
  bool have = false;
  if (src) {
    // The first segment's start state: a copy of the initial state, which the full
    // pass reads instead of init_state (final_state, written by the sequence's last
    // segment in that pass, may alias init_state).
    float *dst = starts + ((int64_t)segi * Hv + h) * kD * kD;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      hreg[j] = src[row * kD + col0 + j];
      dst[row * kD + col0 + j] = hreg[j];
    }
    have = true;
  }
  // the maps' slots and zero flags, 256 segments at a time, loaded in parallel
  __shared__ int sMap[256], sZero[256];
  for (int sb = 0; sb + 1 < s0.nseg; sb += 256) {
    const int nb = min(256, s0.nseg - 1 - sb);
    __syncthreads();  // previous batch consumed
    if (tid < nb) {
      const int m = one_seq ? sb + tid : segs[segi + sb + tid].map;
      sMap[tid] = m;
      sZero[tid] = map_zero[(int64_t)m * Hv + h];
    }
    __syncthreads();
    for (int s = sb; s < sb + nb; ++s) {
      const int64_t m = sMap[s - sb];
      const float *B = maps + ((m * Hv + h) * 2 + 1) * kD * kD;
      if (sZero[s - sb]) {  // H_{s+1} = B_s
        src = B;
        have = false;
        continue;
      }
      if (!have) {
#pragma unroll
        for (int j = 0; j < 8; ++j) hreg[j] = src ? src[row * kD + col0 + j] : 0.f;
        have = true;
      }
      const float *A = maps + ((m * Hv + h) * 2 + 0) * kD * kD;
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
      float *dst = starts + ((int64_t)(segi + s + 1) * Hv + h) * kD * kD;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        hreg[j] = acc[j];
        dst[row * kD + col0 + j] = acc[j];
      }
    }
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

// Segment length: a power of two >= 256 (at most 8192 tokens).  One sequence: the
// smallest that still gives about one round of workgroups over all v heads (512 v-head
// segments: 256 workgroups of two heads, or two of one per compute unit); its segments
// are equal.  Packed sequences of unknown, different lengths: the smallest that gives
// about three rounds, so that the longest-first order of the full pass can fill the last
// round with short segments (the host knows only N and T).  Measured with 16/32 heads:
// 64 sequences of 128-32768 tokens 5.33 ms (one-round rule 5.33, 2048-token cap 5.66);
// five sequences of 500-45000 tokens 1.41 ms (one-round rule 1.65); equal-length
// batches of 2-16 sequences 0.95-0.98 ms (one-round rule 0.92-0.96).
static int32_t pick_seg_len(int64_t T, int32_t Hv, int32_t N) {
  const int64_t target = T * (int64_t)Hv / (N > 1 ? 1536 : 512);
  int32_t s = 256;
  while (s < 8192 && s < target) s *= 2;
  return s;
}

PrefillPlan make_plan(int32_t num_seqs, int64_t total_tokens, int32_t num_v_heads) {
  PrefillPlan p;
  p.num_seqs = num_seqs;
  p.total_tokens = total_tokens;
  p.num_v_heads = num_v_heads;
  if (num_seqs <= 0) return p;
  p.seg_len = pick_seg_len(total_tokens, num_v_heads, num_seqs);
  // sum_i max(1, ceil(L_i / s)) <= N + T / s; segments that are not the last of
  // their sequence are full, so there are at most T / s of them.
  p.max_segments = num_seqs + total_tokens / p.seg_len;
  p.max_maps = total_tokens / p.seg_len;
  const size_t DD = (size_t)kD * kD * sizeof(float);
  size_t off = 0;
  p.off_table = off;
  off = align256(off + sizeof(int32_t) * 16 + sizeof(SegInfo) * (size_t)p.max_segments +
                 sizeof(int32_t) * (size_t)(p.max_maps + 1) + sizeof(int32_t) * (size_t)num_seqs +
                 sizeof(int32_t) * (size_t)p.max_segments);
  if (p.max_maps > 0) {
    p.off_maps = off;
    off = align256(off + 2 * DD * (size_t)p.max_maps * num_v_heads);
    p.off_start = off;
    off = align256(off + DD * (size_t)p.max_segments * num_v_heads);
    p.off_flags = off;
    off = align256(off + sizeof(int32_t) * (size_t)p.max_maps * num_v_heads);
  }
  p.workspace_bytes = off;
  return p;
}

template <typename T>
static hipError_t launch_typed(const PrefillPlan &plan, PrefillArgs args, const int32_t *cu,
                               int N, int64_t Ttot, void *conv_out, hipStream_t stream,
                               PrefillTiming *tm) {
  const int Hv = args.Hv;
  // the full pass runs two v heads per workgroup (one shared q/k prologue) when the
  // v heads of a q/k head pair up
  const bool pairs = (Hv / args.Hk) % 2 == 0;
  static std::atomic<uint64_t> lds_set[3];
  const void *full_fn = pairs ? (const void *)chunk_kernel<T, kFull, 2>
                              : (const void *)chunk_kernel<T, kFull, 1>;
  const int full_lds = pairs ? Lds<2>::BYTES : Lds<1>::BYTES;
  if (hipError_t e = ensure_lds_limit(full_fn, full_lds, lds_set[pairs ? 2 : 0]); e != hipSuccess)
    return e;
  if (hipError_t e = ensure_lds_limit((const void *)chunk_kernel<T, kMap, 1>, Lds<1>::BYTES,
                                      lds_set[1]);
      e != hipSuccess)
    return e;
  auto mark = [&](int slot) {  // event after kernel slot-1 (slot 0 = start)
    if (tm) (void)hipEventRecord(tm->ev[slot], stream);
  };
  // slots: 0 segment table, 1 segment maps (both halves, one launch), 2 combine,
  // 3 full pass, 4 conv-state copy
  if (tm) for (int i = 0; i < kTimedKernels; ++i) tm->ran[i] = false;
  if (tm) tm->ran[0] = !args.one_seq;  // the segment table (launched by the caller)
  mark(1);
  // grids cover ceil(units * Hk / 8) * 8 * r / NH ids (see the id mapping in chunk_kernel)
  auto ids = [&](int64_t units, int nh) {
    const int64_t n = units * args.Hk;
    return ((n + 7) / 8) * 8 * (Hv / args.Hk / nh);
  };
  if (plan.max_maps > 0) {
    dim3 g1((unsigned)(ids(plan.max_maps, 1) * 2));
    hipLaunchKernelGGL((chunk_kernel<T, kMap, 1>), g1, dim3(kThreads), Lds<1>::BYTES, stream, args);
    mark(2);
    dim3 g2((unsigned)((int64_t)N * Hv * 8));
    hipLaunchKernelGGL(combine_kernel, g2, dim3(256), 0, stream, args.segs, args.hdr,
                       args.seq_first, N, args.init_state, (const float *)args.maps,
                       args.map_zero, args.starts, Hv, args.one_seq, args.seg_len, args.T,
                       args.cu);
    mark(3);
    if (tm) tm->ran[1] = tm->ran[2] = true;
  } else {
    mark(2);
    mark(3);
  }
  if (pairs)
    hipLaunchKernelGGL((chunk_kernel<T, kFull, 2>), dim3((unsigned)ids(plan.max_segments, 2)),
                       dim3(2 * kThreads), Lds<2>::BYTES, stream, args);
  else
    hipLaunchKernelGGL((chunk_kernel<T, kFull, 1>), dim3((unsigned)ids(plan.max_segments, 1)),
                       dim3(kThreads), Lds<1>::BYTES, stream, args);
  mark(4);
  if (tm) tm->ran[3] = true;
  if (conv_out) {
    const int64_t n = (int64_t)N * args.Cc;
    hipLaunchKernelGGL((conv_out_kernel<T>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       stream, cu, N, Ttot, (const T *)args.q, (const T *)args.k,
                       (const T *)args.v, (const T *)args.conv_in, (T *)conv_out, args.Hk,
                       args.Hv, args.Cc);
    if (tm) tm->ran[4] = true;
  }
  mark(5);
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
  int32_t *seq_first = map_seg + plan.max_maps + 1;
  int32_t *order = seq_first + num_seqs;
  // One sequence needs no table: every kernel forms the records it reads (seg_record),
  // takes units in order and checks a given cu_seqlens itself.
  const bool one_seq = num_seqs == 1;
  if (!one_seq)
    hipLaunchKernelGGL(segment_table_kernel, dim3(1), dim3(1024), 0, stream, cu_seqlens,
                       num_seqs, total_tokens, plan.seg_len, plan.max_segments, plan.max_maps,
                       segs, hdr, map_seg, seq_first, order);
  PrefillArgs A;
  A.q = q; A.k = k; A.v = v; A.z = z; A.a = a; A.b = b;
  A.conv_w = p.conv_weight; A.A_log = p.A_log; A.dt_bias = p.dt_bias; A.norm_w = p.norm_weight;
  A.q_scale = p.q_scale; A.l2_eps = p.l2_eps; A.rms_eps = p.rms_eps;
  A.init_state = init_state; A.conv_in = conv_state_in; A.o = o; A.final_state = final_state;
  A.segs = segs; A.hdr = hdr; A.map_seg = map_seg; A.seq_first = seq_first; A.order = order;
  A.maps = plan.max_maps > 0 ? (float *)(ws + plan.off_maps) : nullptr;
  A.starts = plan.max_maps > 0 ? (float *)(ws + plan.off_start) : nullptr;
  A.map_zero = plan.max_maps > 0 ? (int32_t *)(ws + plan.off_flags) : nullptr;
  A.Hk = p.num_qk_heads; A.Hv = p.num_v_heads;
  A.gate = p.output_gate;
  A.Cc = 2LL * p.num_qk_heads * kD + (int64_t)p.num_v_heads * kD;
  A.one_seq = one_seq ? 1 : 0;
  A.seg_len = plan.seg_len;
  A.T = (int)total_tokens;
  A.cu = cu_seqlens;
  if (p.act_dtype == GDN_BF16)
    return launch_typed<bf16_t>(plan, A, cu_seqlens, num_seqs, total_tokens, conv_state_out,
                                stream, tm);
  return launch_typed<float>(plan, A, cu_seqlens, num_seqs, total_tokens, conv_state_out, stream,
                             tm);
}

}  // namespace gdn
