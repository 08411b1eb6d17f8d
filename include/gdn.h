/*
 * gdn.h -- C ABI of the MI355X (gfx950) Gated DeltaNet token mixer.
 *
 * The mixer (sources: "Qwen3.8-Flash-Next" tech report, Fig. 2 caption;
 * "Qwen3-Next 80B-A3B" field guide, cutaway 02 "Gated DeltaNet state update";
 * "Qwen3.8-Flash-Next" model card, gated-DeltaNet entry):
 *   x_t   = SiLU(depthwise causal conv, width 4, of the raw q|k|v channels)
 *   q, k  <- L2-normalised per head (q also multiplied by q_scale)
 *   g_t   = -exp(A_log[h]) * softplus(a_t + dt_bias[h]),  alpha_t = exp(g_t)
 *   beta_t = sigmoid(b_t)
 *   S'    = alpha_t S;  e = v_t - S' k_t;  S = S' + beta_t e k_t^T;  y_t = S q_t
 *   o_t   = y_t * rsqrt(mean(y_t^2) + rms_eps) * norm_weight * SiLU(z_t)
 *           (or * sigmoid(z_t) with params->output_gate = GDN_GATE_SIGMOID)
 * with Hk q/k heads, Hv v heads (v head h reads q/k head h / (Hv/Hk)), head
 * dim D = 128, one D x D fp32 state per (sequence, v head).
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers to dense row-major memory unless a
 *     name ends in _host.  The caller owns every buffer (workspace included);
 *     the library keeps no pointer after a call returns.  Buffers must stay
 *     alive until `stream` has finished the enqueued work.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = default stream)
 *     without host synchronisation, except where a function says otherwise.
 *   - Activation tensors (q, k, v, z, o, conv state) have dtype
 *     params->act_dtype (bf16 or fp32).  Gates a, b, parameters and states are
 *     fp32.  bf16 stores round to nearest even.
 *   - The state of one (sequence, v head) is stored as H = S^T, i.e. a
 *     [D][D] block whose row index is the key dim and column index the value
 *     dim (the model card's state[dk][dv] layout).
 *   - The conv state of one sequence is [3][Cc] raw inputs, oldest row first,
 *     Cc = 2*Hk*D + Hv*D channels in the order q | k | v (channel = section
 *     offset + head*D + i).  Tap 3 of conv_weight multiplies the current
 *     token, tap 0 the token three steps back.
 *   - Errors: argument problems the host can see are reported before anything
 *     is enqueued, and then no output is modified.  A failed launch returns
 *     GDN_ERR_HIP.  gdn_last_error() gives a thread-local message for the last
 *     failing call.  NaN/Inf in inputs are propagated, not checked.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GDN_BF16 = 0, GDN_F32 = 1 } gdn_dtype;

/* Output gate of the epilogue: SiLU(z) (the field guide's, the default) or
 * sigmoid(z) (the variant the tech report's Fig. 2 caption starts to name). */
typedef enum { GDN_GATE_SILU = 0, GDN_GATE_SIGMOID = 1 } gdn_gate;

typedef enum {
  GDN_OK = 0,
  GDN_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, bad layout */
  GDN_ERR_UNSUPPORTED = 2,      /* valid but not built: head_dim != 128, ... */
  GDN_ERR_WORKSPACE = 3,        /* workspace missing or smaller than required */
  GDN_ERR_NO_DEVICE = 4,        /* no usable gfx950 device */
  GDN_ERR_HIP = 5               /* a HIP runtime call or launch failed */
} gdn_status;

/* Mixer parameters.  The struct itself is host memory read during the call;
 * the weight pointers are device pointers. */
typedef struct {
  int32_t num_qk_heads;       /* Hk >= 1 */
  int32_t num_v_heads;        /* Hv, a multiple of Hk */
  int32_t head_dim;           /* D; the kernels are built for D = 128 */
  int32_t act_dtype;          /* gdn_dtype of q, k, v, z, o and conv state */
  float q_scale;              /* multiplies q after L2 normalisation (1.0) */
  float l2_eps;               /* x / sqrt(sum x^2 + l2_eps) (1e-6) */
  float rms_eps;              /* y * rsqrt(mean y^2 + rms_eps) (1e-6) */
  const float *conv_weight;   /* [Cc][4] */
  const float *A_log;         /* [Hv] */
  const float *dt_bias;       /* [Hv] */
  const float *norm_weight;   /* [D], or NULL for all ones */
  int32_t output_gate;        /* gdn_gate: o = RMSNorm(y) * norm_weight * gate(z) */
} gdn_params;

/* Bytes of device workspace gdn_prefill needs for this problem (0 is a valid
 * answer).  Depends only on the parameters, num_seqs and total_tokens.
 * Returns (size_t)-1 for invalid arguments. */
size_t gdn_prefill_workspace_bytes(const gdn_params *p, int32_t num_seqs,
                                   int64_t total_tokens);

/* Chunked prefill of num_seqs packed sequences (the whole mixer; the state
 * update follows the model card's chunk form state*chunk_decay + key^T v_new,
 * with chunks of 32 tokens aligned to each sequence's start).
 *
 *   q, k          [T, Hk, D] act dtype        T = total_tokens
 *   v, z          [T, Hv, D] act dtype
 *   a, b          [T, Hv] fp32
 *   init_state    [N, Hv, D, D] fp32, or NULL for zeros
 *   cu_seqlens    [N+1] int32 device: cu[0] = 0, non-decreasing, cu[N] = T;
 *                 may be NULL when N = 1.  The host does not read the contents
 *                 (no synchronisation); the first kernel checks them on the
 *                 device, and for an invalid table runs nothing else (o and
 *                 final_state are left unwritten) and sets a per-device error
 *                 flag that gdn_check_device_errors() reports.  With the
 *                 environment variable GDN_VALIDATE=1 the call instead
 *                 synchronises, reports a flag left by an earlier call, copies
 *                 cu_seqlens to the host and checks it before launching.
 *                 Zero-length sequences are allowed: their final state equals
 *                 their initial state bit for bit.
 *   conv_state_in [N, 3, Cc] act dtype, or NULL for zeros
 *   o             [T, Hv, D] act dtype (out); must not alias an input
 *   final_state   [N, Hv, D, D] fp32 (out); may alias init_state (a sequence
 *                 split over several workgroups starts from a copy of its
 *                 initial state taken in the workspace before any final state
 *                 is written)
 *   conv_state_out[N, 3, Cc] act dtype (out), or NULL; may alias conv_state_in
 *   workspace     device memory of at least gdn_prefill_workspace_bytes()
 *                 bytes (may be NULL when that is 0), 256-byte aligned.
 */
gdn_status gdn_prefill(const void *q, const void *k, const void *v,
                       const float *a, const float *b, const void *z,
                       const gdn_params *p, const float *init_state,
                       const int32_t *cu_seqlens, int32_t num_seqs,
                       int64_t total_tokens, const void *conv_state_in,
                       void *o, float *final_state, void *conv_state_out,
                       void *workspace, size_t workspace_bytes, void *stream);

/* Largest workspace, in bytes, that gdn_prefill_noalloc can use. */
#define GDN_NOALLOC_WORKSPACE_BYTES ((size_t)128 << 20)

/* gdn_prefill for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Arguments, results
 * and errors are those of gdn_prefill without the workspace: the library uses its own
 * static device array of GDN_NOALLOC_WORKSPACE_BYTES per device, which is part of
 * the library's code object and stays allocated until the process ends.
 *   - Returns GDN_ERR_WORKSPACE, before anything is enqueued, when
 *     gdn_prefill_workspace_bytes() for the problem exceeds that size (one sequence
 *     of up to 131072 tokens at 32 v heads fits; large varlen batches may not).
 *   - Performs no allocation (no hipMalloc, hipFree or host buffer) and no host
 *     synchronisation after its first call on a device, which looks the array's
 *     device address up; GDN_VALIDATE and GDN_KERNEL_TIMING are ignored.
 *   - Every call on one device shares that device's array, which keeps the last
 *     call's contents (nothing in it needs to start at zero).  Calls that may
 *     overlap on one device (on streams not ordered with each other) race, and
 *     must not be issued. */
gdn_status gdn_prefill_noalloc(const void *q, const void *k, const void *v,
                               const float *a, const float *b, const void *z,
                               const gdn_params *p, const float *init_state,
                               const int32_t *cu_seqlens, int32_t num_seqs,
                               int64_t total_tokens, const void *conv_state_in,
                               void *o, float *final_state, void *conv_state_out,
                               void *stream);

/* Reports, and clears, an error that a kernel of an earlier call on the current
 * device found in device-resident arguments: today an invalid cu_seqlens table
 * passed to gdn_prefill or gdn_gated_attention (GDN_ERR_INVALID_ARGUMENT).  Synchronises `stream` first
 * (host synchronisation).  GDN_OK when no such error is pending. */
gdn_status gdn_check_device_errors(void *stream);

/* One decode step (one new token) for `batch` independent sequences: the
 * field guide's six update operations applied once per (sequence, v head),
 * reading and writing each fp32 state exactly once.
 *
 *   q, k        [B, Hk, D] act dtype;  v, z [B, Hv, D] act dtype
 *   a, b        [B, Hv] fp32
 *   state       [B, Hv, D, D] fp32, updated in place
 *   conv_state  [B, 3, Cc] act dtype, updated in place to the last three raw
 *               inputs (oldest first)
 *   o           [B, Hv, D] act dtype (out)
 * Not transactional: a caller that needs rollback keeps a copy of
 * (state, conv_state). */
gdn_status gdn_decode_step(const void *q, const void *k, const void *v,
                           const float *a, const float *b, const void *z,
                           const gdn_params *p, float *state, void *conv_state,
                           void *o, int32_t batch, void *stream);

/* gdn_decode_step with the state stored in bf16: state is [B, Hv, D, D] bf16
 * (uint16 bit patterns), read once per step, widened to fp32 for the step's
 * arithmetic (identical to gdn_decode_step's), and written back rounded to
 * nearest even.  Halves the state bytes that dominate a decode step.  This is a
 * reduced-precision storage mode beside the pages' fp32 state: the stored state
 * carries one bf16 rounding per step (its own tolerance; see the tests).  Other
 * arguments and errors as gdn_decode_step. */
gdn_status gdn_decode_step_bf16_state(const void *q, const void *k, const void *v,
                                      const float *a, const float *b, const void *z,
                                      const gdn_params *p, void *state, void *conv_state,
                                      void *o, int32_t batch, void *stream);

/* gdn_decode_step with the state stored in fp8: state is [B, Hv, D, D] OCP E4M3
 * bytes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; largest finite value
 * 448) and state_scale [B, Hv, D] fp32 holds one power-of-two scale per state row
 * (per dk index i of H = S^T): the stored state is H[i][j] = e4m3(state[i][j]) *
 * state_scale[i].  Each step reads both once, does the step's arithmetic in fp32
 * (identical to gdn_decode_step's), and writes back every row re-scaled by the
 * smallest power of two 2^e with max_j |H[i][j]| <= 448 * 2^e (1 for a zero row)
 * and rounded to nearest even.  A quarter of the fp32 state's bytes; a
 * reduced-precision storage mode beside the pages' fp32 state (one fp8 rounding per
 * step: its own tolerance, see the tests).  Other arguments and errors as
 * gdn_decode_step; state_scale is required (GDN_ERR_INVALID_ARGUMENT). */
gdn_status gdn_decode_step_fp8_state(const void *q, const void *k, const void *v,
                                     const float *a, const float *b, const void *z,
                                     const gdn_params *p, void *state, float *state_scale,
                                     void *conv_state, void *o, int32_t batch, void *stream);

/* n_tokens new tokens per sequence on a cached state (multi-token decode; the
 * verify and commit passes of speculative decoding).  The result is that of
 * n_tokens gdn_decode_step calls in order (the field guide's six update
 * operations per token, cutaway 02), but each fp32 state is read once and
 * written at most once for all n_tokens.
 *
 *   q, k        [B, n, Hk, D] act dtype;  v, z [B, n, Hv, D] act dtype
 *   a, b        [B, n, Hv] fp32
 *   state       [B, Hv, D, D] fp32, in/out
 *   conv_state  [B, 3, Cc] act dtype, in/out (oldest row first)
 *   num_commit  [B] int32 device, or NULL: the state and the conv cache of
 *               sequence b advance by num_commit[b] tokens (values are clamped
 *               to 0..n; NULL means n for every sequence).  With 0 neither is
 *               written (a verify pass); a later call with the accepted count
 *               advances them.
 *   o           [B, n, Hv, D] act dtype (out): outputs of all n tokens, token t
 *               seeing tokens 0..t of this call whatever num_commit says
 *   1 <= n_tokens <= 8.  Not transactional (as gdn_decode_step). */
gdn_status gdn_decode_tokens(const void *q, const void *k, const void *v,
                             const float *a, const float *b, const void *z,
                             const gdn_params *p, float *state, void *conv_state,
                             const int32_t *num_commit, void *o, int32_t batch,
                             int32_t n_tokens, void *stream);

/* ---- Projections around the mixer (token-parallel linear layers) ----------------
 * The mixer's q, k, v, z, a, b are projections of the hidden states, and its gated
 * output is projected back ("Qwen3.8-Flash-Next" tech report, Fig. 2 caption: the
 * projected query, key and value streams; "Qwen3-Next 80B-A3B" field guide, cutaway
 * 02: the output is gated and projected).  All three run one bf16 MFMA GEMM kernel,
 * y = x w^T with fp32 accumulation: x [M, K] bf16 row-major (one token per row), w
 * [N, K] bf16 row-major (one row of weights per output feature, the layout of a
 * linear layer's weight matrix), K a multiple of 64 (GDN_ERR_UNSUPPORTED otherwise).
 * Outputs are rounded to nearest even where they are bf16. */

/* y [M, N] bf16 = x w^T. */
gdn_status gdn_linear(const void *x, const void *w, int64_t M, int32_t N, int32_t K, void *y,
                      void *stream);

/* The mixer's input projection, written straight into the tensors gdn_prefill reads:
 * x [T, d_model] bf16, w_in [N_in, d_model] bf16 with N_in = 2*Hk*D + 2*Hv*D + 2*Hv, its
 * rows in the order q (Hk*D rows, head-major), k (Hk*D), v (Hv*D), z (Hv*D), a (Hv),
 * b (Hv).  q, k [T, Hk, D] and v, z [T, Hv, D] in p->act_dtype; a, b [T, Hv] fp32.
 * (Only the head counts, head_dim and act_dtype of p are used.) */
gdn_status gdn_in_projection(const void *x, const void *w_in, const gdn_params *p, int64_t T,
                             int32_t d_model, void *q, void *k, void *v, void *z, float *a,
                             float *b, void *stream);

/* The output projection: y [T, d_model] bf16 = o w_out^T with o [T, Hv, D] bf16 read as
 * [T, Hv*D] and w_out [d_model, Hv*D] bf16.  p->act_dtype must be GDN_BF16. */
gdn_status gdn_out_projection(const void *o, const void *w_out, const gdn_params *p, int64_t T,
                              int32_t d_model, void *y, void *stream);

/* ---- The hybrid's gated full-attention layer ------------------------------------
 * Every fourth mixer of the hybrid is softmax attention ("Qwen3-Next 80B-A3B" field
 * guide, cutaway 03: grouped queries, 16 query heads over 2 key/value heads, head dim
 * 256, rotary embedding on the first 64 dims, QK-Norm, a sigmoid output gate;
 * "Qwen3.8-Flash-Next" model card, attention entries: per-head RMSNorm of q and k
 * before the rotation, the rotate/nope split, the output times sigmoid of the gate):
 *   q^ = RoPE(RMSNorm(q) * q_norm_weight),  k^ = RoPE(RMSNorm(k) * k_norm_weight)
 *   o  = softmax(causal(q^ k^T * scale)) v * sigmoid(gate)
 * RMSNorm(x) = x / sqrt(mean(x^2) + norm_eps) over the head dim.  RoPE rotates the
 * pair (i, i + rotary_dim/2), i < rotary_dim/2, by pos * rope_theta^(-2i/rotary_dim),
 * pos counted from 0 at each sequence's first token; dims >= rotary_dim pass through.
 * Query head h reads key/value head h / (Hq / Hkv).  Queries attend to the keys of
 * their own sequence up to and including their own position. */
typedef struct {
  int32_t num_q_heads;           /* Hq, a multiple of num_kv_heads */
  int32_t num_kv_heads;          /* Hkv >= 1 */
  int32_t head_dim;              /* the kernels are built for 256 */
  int32_t rotary_dim;            /* 0 <= rotary_dim <= head_dim, a multiple of 16 (64) */
  float rope_theta;              /* > 0 (10000) */
  float norm_eps;                /* >= 0 (1e-6) */
  float scale;                   /* softmax scale; <= 0 selects head_dim^-1/2 */
  const float *q_norm_weight;    /* [head_dim] device fp32, or NULL for all ones */
  const float *k_norm_weight;    /* [head_dim] device fp32, or NULL for all ones */
} gdn_attn_params;

/* Bytes of device workspace gdn_gated_attention needs (2 * T * (Hq + Hkv) * head_dim
 * plus 512 at most); (size_t)-1 for invalid arguments. */
size_t gdn_gated_attention_workspace_bytes(const gdn_attn_params *p, int64_t total_tokens);

/* Causal gated attention over num_seqs packed sequences, bf16 in and out:
 *   q, gate      [T, Hq, head_dim] bf16          T = total_tokens
 *   k, v         [T, Hkv, head_dim] bf16
 *   cu_seqlens   [N+1] int32 device, as for gdn_prefill (NULL allowed when N = 1).  The
 *                first kernel checks the table on the device; for an invalid one no
 *                output is written and gdn_check_device_errors() reports the error.
 *                GDN_VALIDATE=1 makes the call check it on the host first
 *                (synchronising), as gdn_prefill does.
 *   o            [T, Hq, head_dim] bf16 (out); must not alias an input
 *   workspace    at least gdn_gated_attention_workspace_bytes() bytes, 256-byte
 *                aligned (holds the normalised, rotated q^ and k^ in fp16).
 * Errors: GDN_ERR_UNSUPPORTED for head_dim != 256 or T * (Hq + Hkv) >= 2^27;
 * GDN_ERR_INVALID_ARGUMENT for bad sizes, rotary_dim, theta or pointers. */
gdn_status gdn_gated_attention(const void *q, const void *k, const void *v, const void *gate,
                               const gdn_attn_params *p, const int32_t *cu_seqlens,
                               int32_t num_seqs, int64_t total_tokens, void *o,
                               void *workspace, size_t workspace_bytes, void *stream);

/* Diagnostics: per-kernel device time of the last gdn_prefill call made on
 * this thread while the environment had GDN_KERNEL_TIMING=1.  The library then
 * records HIP events on the caller's stream between its kernels (segment table,
 * segment-map pass, combine, full pass, conv-state copy).  Writes up to
 * `max_kernels` milliseconds (0 for a kernel that did not run) and returns the
 * number of slots written, or -1 when there is no timed call.  Waits for the
 * timed call's last event (host synchronisation). */
int gdn_prefill_last_kernel_times(float *ms, int max_kernels);

/* Static text for a status code. */
const char *gdn_status_string(gdn_status s);

/* Thread-local detail message of the last failing call on this thread
 * ("" if none). */
const char *gdn_last_error(void);

/* Library version string. */
const char *gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
