/*
 * gdn_oracle.c -- plain fp64 CPU oracle of the Gated DeltaNet token mixer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke entry and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header
 * or constant with the GPU library and is never a fallback for it.
 *
 * What it computes (sources are the pages this project is built from):
 *   - "Qwen3.8-Flash-Next" tech report, Fig. 2 caption: projected q/k/v pass
 *     through short causal convolutions; q and k are L2-normalised before the
 *     gated delta recurrence; a decay gate alpha_t and a write gate beta_t
 *     control the update.
 *   - "Qwen3-Next 80B-A3B" field guide, cutaway 02 "Gated DeltaNet state
 *     update" (technical read and the six numbered operations): 16 q/k heads,
 *     32 v/state/gate heads, head width 128, width-4 depthwise causal conv;
 *     S maps key -> value; S' = decay*S, vhat = S'k, e = v - vhat,
 *     S'' = S' + (beta e) k^T, y = S'' q; then RMS-normalise y and gate it
 *     with SiLU(z).
 *   - "Qwen3.8-Flash-Next" model card, gated-DeltaNet entry: the decay gate
 *     g = -exp(A_log) * softplus(a + dt_bias) per head; alpha = exp(g).
 *   - beta = sigmoid(b) and a SiLU after the conv are the plainest readings
 *     the pages leave open (the caption names beta and the conv but not their
 *     exact forms).
 *
 * Every function below is the plain definition, written token by token with
 * no blocking, chunking or reordering.  All arithmetic is fp64; inputs are the
 * exact values of the (bf16 or fp32) tensors the GPU path receives.
 *
 * Layouts (row-major):
 *   q, k    [T, Hk, D]       v, z [T, Hv, D]       a, b [T, Hv]
 *   conv_w  [Cc][4], Cc = 2*Hk*D + Hv*D, channel order q | k | v,
 *           channel index = section offset + head*D + i; tap 3 multiplies the
 *           current token, tap 0 the token three steps back.
 *   conv history [N][3][Cc], oldest row first.
 *   state   [N, Hv, D, D] stored as H = S^T, i.e. H[i][j] = S[j][i]
 *           (row index = key dim, column index = value dim).
 *   v head h reads q/k head h / (Hv/Hk).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- scalars */

double oracle_sigmoid(double u) { return 1.0 / (1.0 + exp(-u)); }

double oracle_silu(double u) { return u * oracle_sigmoid(u); }

/* softplus(u) = log(1 + e^u), written so that it neither overflows nor loses
 * the small-|u| digits. */
double oracle_softplus(double u) {
  double m = u > 0.0 ? u : 0.0;
  return m + log1p(exp(-fabs(u)));
}

/* Decay and write gates of one (token, v head): model card, gated-DeltaNet
 * entry (g), Fig. 2 caption (alpha_t, beta_t). */
void oracle_gates(int64_t n, const double *a, const double *b, double A_log,
                  double dt_bias, double *alpha, double *beta) {
  double decay_rate = exp(A_log);
  for (int64_t t = 0; t < n; ++t) {
    double g = -decay_rate * oracle_softplus(a[t] + dt_bias);
    alpha[t] = exp(g);
    beta[t] = oracle_sigmoid(b[t]);
  }
}

/* ------------------------------------------------------------- prologue */

/* Width-4 depthwise causal conv of one channel over one sequence followed by
 * SiLU.  x[t*stride] are the raw inputs of this channel, hist[0..2] the three
 * raw values before the sequence (oldest first), w[0..3] the taps. */
static void conv_silu_channel(int64_t T, const double *x, int64_t stride,
                              const double hist[3], const double w[4],
                              double *out, int64_t out_stride) {
  for (int64_t t = 0; t < T; ++t) {
    double acc = 0.0;
    for (int j = 0; j < 4; ++j) {
      int64_t tau = t - 3 + j; /* token this tap reads */
      double xv = tau >= 0 ? x[tau * stride] : hist[3 + tau];
      acc += w[j] * xv;
    }
    out[t * out_stride] = oracle_silu(acc);
  }
}

/* Prologue of one (sequence, v head) unit: post-conv, post-SiLU q and k of
 * q/k head g (L2-normalised, q also scaled) and v of v head h.
 * Outputs are [T][D] each. */
void oracle_prologue(int64_t T, int Hk, int Hv, int D, int h,
                     const double *q, const double *k, const double *v,
                     const double *conv_w, const double *hist /* [3][Cc] or NULL */,
                     double q_scale, double l2_eps,
                     double *qo, double *ko, double *vo) {
  int r = Hv / Hk;
  int g = h / r;
  int64_t Cc = 2LL * Hk * D + (int64_t)Hv * D;
  int64_t cq = (int64_t)g * D, ck = (int64_t)Hk * D + (int64_t)g * D,
          cv = 2LL * Hk * D + (int64_t)h * D;
  for (int i = 0; i < D; ++i) {
    double hq[3] = {0, 0, 0}, hk[3] = {0, 0, 0}, hv[3] = {0, 0, 0};
    if (hist) {
      for (int j = 0; j < 3; ++j) {
        hq[j] = hist[j * Cc + cq + i];
        hk[j] = hist[j * Cc + ck + i];
        hv[j] = hist[j * Cc + cv + i];
      }
    }
    conv_silu_channel(T, q + (int64_t)g * D + i, (int64_t)Hk * D, hq,
                      conv_w + (cq + i) * 4, qo + i, D);
    conv_silu_channel(T, k + (int64_t)g * D + i, (int64_t)Hk * D, hk,
                      conv_w + (ck + i) * 4, ko + i, D);
    conv_silu_channel(T, v + (int64_t)h * D + i, (int64_t)Hv * D, hv,
                      conv_w + (cv + i) * 4, vo + i, D);
  }
  /* L2 normalisation of q and k per token (Fig. 2 caption). */
  for (int64_t t = 0; t < T; ++t) {
    double sq = 0.0, sk = 0.0;
    for (int i = 0; i < D; ++i) {
      sq += qo[t * D + i] * qo[t * D + i];
      sk += ko[t * D + i] * ko[t * D + i];
    }
    double fq = q_scale / sqrt(sq + l2_eps), fk = 1.0 / sqrt(sk + l2_eps);
    for (int i = 0; i < D; ++i) {
      qo[t * D + i] *= fq;
      ko[t * D + i] *= fk;
    }
  }
}

/* ----------------------------------------------------------- recurrence */

/* The gated delta recurrence of one head, in the field guide's column-vector
 * convention (S maps key -> value), steps 1-6 of its cutaway 02 in order:
 *   S' = alpha_t S;  vhat = S' k_t;  e = v_t - vhat;  S = S' + (beta_t e) k_t^T;
 *   y_t = S q_t.
 * S is [D][D] with S[row = value dim][col = key dim]; it is updated in place.
 * q, k, v, y are [T][D]. */
void oracle_recurrence(int64_t T, int D, const double *alpha, const double *beta,
                       const double *q, const double *k, const double *v,
                       double *S, double *y) {
  double *vhat = (double *)malloc(sizeof(double) * D);
  for (int64_t t = 0; t < T; ++t) {
    const double *kt = k + t * D, *qt = q + t * D, *vt = v + t * D;
    /* 1. decay the old state */
    for (int64_t e = 0; e < (int64_t)D * D; ++e) S[e] *= alpha[t];
    /* 2. read the current association */
    for (int r = 0; r < D; ++r) {
      double acc = 0.0;
      for (int c = 0; c < D; ++c) acc += S[r * D + c] * kt[c];
      vhat[r] = acc;
    }
    /* 3-5. measure the error, gate it, write error (x) key */
    for (int r = 0; r < D; ++r) {
      double be = beta[t] * (vt[r] - vhat[r]);
      for (int c = 0; c < D; ++c) S[r * D + c] += be * kt[c];
    }
    /* 6. read with the query */
    for (int r = 0; r < D; ++r) {
      double acc = 0.0;
      for (int c = 0; c < D; ++c) acc += S[r * D + c] * qt[c];
      y[t * D + r] = acc;
    }
  }
  free(vhat);
}

/* ------------------------------------------------------------- epilogue */

/* Output gate: 0 = SiLU(z) (field guide cutaway 02, last line), 1 = sigmoid(z)
 * (the variant the tech report's Fig. 2 caption starts to name, "while a sigmoid
 * ...", and the form of the model card's attention output gate). */
static double output_gate(int gate, double z) {
  return gate == 1 ? oracle_sigmoid(z) : oracle_silu(z);
}

/* Output of one head: RMS-normalise y over the head's D values, scale by the norm
 * weight, multiply by the output gate of z.  y, z, o are [T][D] with z and o
 * strided by z_stride / o_stride per token. */
void oracle_epilogue_gated(int64_t T, int D, const double *y, const double *z,
                           int64_t z_stride, const double *norm_w /* [D] or NULL */,
                           double rms_eps, double *o, int64_t o_stride, int gate) {
  for (int64_t t = 0; t < T; ++t) {
    double ss = 0.0;
    for (int i = 0; i < D; ++i) ss += y[t * D + i] * y[t * D + i];
    double inv = 1.0 / sqrt(ss / D + rms_eps);
    for (int i = 0; i < D; ++i) {
      double w = norm_w ? norm_w[i] : 1.0;
      o[t * o_stride + i] = y[t * D + i] * inv * w * output_gate(gate, z[t * z_stride + i]);
    }
  }
}

/* The field guide's epilogue: the SiLU(z) gate. */
void oracle_epilogue(int64_t T, int D, const double *y, const double *z,
                     int64_t z_stride, const double *norm_w, double rms_eps, double *o,
                     int64_t o_stride) {
  oracle_epilogue_gated(T, D, y, z, z_stride, norm_w, rms_eps, o, o_stride, 0);
}

/* ---------------------------------------------------------------- mixer */

typedef struct {
  int N, Hk, Hv, D;
  const int64_t *cu;
  const double *q, *k, *v, *a, *b, *z, *conv_w, *A_log, *dt_bias, *norm_w;
  double q_scale, l2_eps, rms_eps;
  int gate;
  const double *init_state, *conv_in;
  double *o, *final_state;
  int64_t next_unit; /* work counter, taken with an atomic add */
} mixer_job;

/* One (sequence, v head) unit: prologue, recurrence, epilogue, state out. */
static void run_unit(mixer_job *J, int64_t unit) {
  int n = (int)(unit / J->Hv), h = (int)(unit % J->Hv);
  int D = J->D, Hk = J->Hk, Hv = J->Hv;
  int64_t t0 = J->cu[n], T = J->cu[n + 1] - t0;
  int64_t Cc = 2LL * Hk * D + (int64_t)Hv * D;
  double *S = (double *)malloc(sizeof(double) * D * D);
  const double *H0 = J->init_state ? J->init_state + ((int64_t)n * Hv + h) * D * D : NULL;
  for (int i = 0; i < D; ++i)
    for (int j = 0; j < D; ++j) S[j * D + i] = H0 ? H0[i * D + j] : 0.0; /* S = H^T */
  if (T > 0) {
    double *qo = (double *)malloc(sizeof(double) * T * D);
    double *ko = (double *)malloc(sizeof(double) * T * D);
    double *vo = (double *)malloc(sizeof(double) * T * D);
    double *y = (double *)malloc(sizeof(double) * T * D);
    double *al = (double *)malloc(sizeof(double) * T);
    double *be = (double *)malloc(sizeof(double) * T);
    double *at = (double *)malloc(sizeof(double) * T);
    double *bt = (double *)malloc(sizeof(double) * T);
    oracle_prologue(T, Hk, Hv, D, h, J->q + t0 * Hk * D, J->k + t0 * Hk * D,
                    J->v + t0 * Hv * D, J->conv_w,
                    J->conv_in ? J->conv_in + (int64_t)n * 3 * Cc : NULL,
                    J->q_scale, J->l2_eps, qo, ko, vo);
    for (int64_t t = 0; t < T; ++t) {
      at[t] = J->a[(t0 + t) * Hv + h];
      bt[t] = J->b[(t0 + t) * Hv + h];
    }
    oracle_gates(T, at, bt, J->A_log[h], J->dt_bias[h], al, be);
    oracle_recurrence(T, D, al, be, qo, ko, vo, S, y);
    oracle_epilogue_gated(T, D, y, J->z + (t0 * Hv + h) * D, (int64_t)Hv * D, J->norm_w,
                          J->rms_eps, J->o + (t0 * Hv + h) * D, (int64_t)Hv * D, J->gate);
    free(qo); free(ko); free(vo); free(y); free(al); free(be); free(at); free(bt);
  }
  double *Hf = J->final_state + ((int64_t)n * Hv + h) * D * D;
  for (int i = 0; i < D; ++i)
    for (int j = 0; j < D; ++j) Hf[i * D + j] = S[j * D + i];
  free(S);
}

static void *worker(void *arg) {
  mixer_job *J = (mixer_job *)arg;
  int64_t total = (int64_t)J->N * J->Hv;
  for (;;) {
    int64_t u = __atomic_fetch_add(&J->next_unit, 1, __ATOMIC_RELAXED);
    if (u >= total) break;
    run_unit(J, u);
  }
  return NULL;
}

/* Full mixer over N packed sequences.  cu_seqlens [N+1] (cu[0] = 0, monotone).
 * init_state / conv_in may be NULL (zeros).  conv_out [N][3][Cc] (may be NULL)
 * receives the last three raw inputs of each sequence, taking rows from the
 * inherited history when the sequence is shorter than three.
 * gate selects the output gate (0 SiLU(z), 1 sigmoid(z)).
 * Returns 0, or -1 on an invalid argument. */
int oracle_prefill_gated(int N, const int64_t *cu_seqlens, int Hk, int Hv, int D,
                         const double *q, const double *k, const double *v,
                         const double *a, const double *b, const double *z,
                         const double *conv_w, const double *A_log, const double *dt_bias,
                         const double *norm_w, double q_scale, double l2_eps, double rms_eps,
                         const double *init_state, const double *conv_in,
                         double *o, double *final_state, double *conv_out, int nthreads,
                         int gate) {
  if (gate != 0 && gate != 1) return -1;
  if (N < 0 || Hk <= 0 || Hv <= 0 || D <= 0 || Hv % Hk != 0 || !cu_seqlens) return -1;
  if (cu_seqlens[0] != 0) return -1;
  for (int n = 0; n < N; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
  mixer_job J;
  memset(&J, 0, sizeof(J));
  J.N = N; J.Hk = Hk; J.Hv = Hv; J.D = D; J.cu = cu_seqlens;
  J.q = q; J.k = k; J.v = v; J.a = a; J.b = b; J.z = z; J.conv_w = conv_w;
  J.A_log = A_log; J.dt_bias = dt_bias; J.norm_w = norm_w;
  J.q_scale = q_scale; J.l2_eps = l2_eps; J.rms_eps = rms_eps; J.gate = gate;
  J.init_state = init_state; J.conv_in = conv_in; J.o = o; J.final_state = final_state;
  J.next_unit = 0;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  int started = 0;
  for (int i = 1; i < nthreads; ++i)
    if (pthread_create(&th[started], NULL, worker, &J) == 0) ++started;
  worker(&J);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);

  if (conv_out) {
    int64_t Cc = 2LL * Hk * D + (int64_t)Hv * D;
    for (int n = 0; n < N; ++n) {
      int64_t t0 = cu_seqlens[n], T = cu_seqlens[n + 1] - t0;
      for (int row = 0; row < 3; ++row) {
        int64_t tau = T - 3 + row; /* position relative to the sequence start */
        double *dst = conv_out + ((int64_t)n * 3 + row) * Cc;
        for (int64_t c = 0; c < Cc; ++c) {
          double xv;
          if (tau >= 0) {
            int64_t t = t0 + tau;
            if (c < (int64_t)Hk * D) xv = q[t * Hk * D + c];
            else if (c < 2LL * Hk * D) xv = k[t * Hk * D + (c - (int64_t)Hk * D)];
            else xv = v[t * Hv * D + (c - 2LL * Hk * D)];
          } else {
            xv = conv_in ? conv_in[((int64_t)n * 3 + (3 + tau)) * Cc + c] : 0.0;
          }
          dst[c] = xv;
        }
      }
    }
  }
  return 0;
}

/* The mixer with the field guide's SiLU(z) gate. */
int oracle_prefill(int N, const int64_t *cu_seqlens, int Hk, int Hv, int D,
                   const double *q, const double *k, const double *v,
                   const double *a, const double *b, const double *z,
                   const double *conv_w, const double *A_log, const double *dt_bias,
                   const double *norm_w, double q_scale, double l2_eps, double rms_eps,
                   const double *init_state, const double *conv_in,
                   double *o, double *final_state, double *conv_out, int nthreads) {
  return oracle_prefill_gated(N, cu_seqlens, Hk, Hv, D, q, k, v, a, b, z, conv_w, A_log,
                              dt_bias, norm_w, q_scale, l2_eps, rms_eps, init_state, conv_in,
                              o, final_state, conv_out, nthreads, 0);
}

/* One decode step for B independent sequences: exactly one token of the mixer
 * with the conv cache as history, the state updated in place, and the cache
 * shifted to [cache1, cache2, x_t].  Shapes as oracle_prefill with T = B. */
int oracle_decode_step_gated(int B, int Hk, int Hv, int D,
                             const double *q, const double *k, const double *v,
                             const double *a, const double *b, const double *z,
                             const double *conv_w, const double *A_log, const double *dt_bias,
                             const double *norm_w, double q_scale, double l2_eps,
                             double rms_eps, double *state, double *conv_cache, double *o,
                             int nthreads, int gate) {
  if (B < 0) return -1;
  int64_t *cu = (int64_t *)malloc(sizeof(int64_t) * (B + 1));
  for (int i = 0; i <= B; ++i) cu[i] = i;
  int64_t Cc = 2LL * Hk * D + (int64_t)Hv * D;
  double *new_cache = (double *)malloc(sizeof(double) * (size_t)B * 3 * Cc + 1);
  int rc = oracle_prefill_gated(B, cu, Hk, Hv, D, q, k, v, a, b, z, conv_w, A_log, dt_bias,
                                norm_w, q_scale, l2_eps, rms_eps, state, conv_cache, o, state,
                                new_cache, nthreads, gate);
  if (rc == 0) memcpy(conv_cache, new_cache, sizeof(double) * (size_t)B * 3 * Cc);
  free(new_cache);
  free(cu);
  return rc;
}

int oracle_decode_step(int B, int Hk, int Hv, int D,
                       const double *q, const double *k, const double *v,
                       const double *a, const double *b, const double *z,
                       const double *conv_w, const double *A_log, const double *dt_bias,
                       const double *norm_w, double q_scale, double l2_eps, double rms_eps,
                       double *state, double *conv_cache, double *o, int nthreads) {
  return oracle_decode_step_gated(B, Hk, Hv, D, q, k, v, a, b, z, conv_w, A_log, dt_bias,
                                  norm_w, q_scale, l2_eps, rms_eps, state, conv_cache, o,
                                  nthreads, 0);
}
