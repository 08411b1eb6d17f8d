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
 *                 may be NULL when N = 1.  Contents are not validated unless
 *                 the environment sets GDN_VALIDATE=1 (then the call copies
 *                 them to the host synchronously and checks them).
 *                 Zero-length sequences are allowed: their final state equals
 *                 their initial state bit for bit.
 *   conv_state_in [N, 3, Cc] act dtype, or NULL for zeros
 *   o             [T, Hv, D] act dtype (out); must not alias an input
 *   final_state   [N, Hv, D, D] fp32 (out); may alias init_state
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

/* Diagnostics: per-kernel device time of the last gdn_prefill call made on
 * this thread while the environment had GDN_KERNEL_TIMING=1.  The library then
 * records HIP events on the caller's stream between its kernels (segment table,
 * map pass A, map pass B, combine, full pass, conv-state copy).  Writes up to
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
