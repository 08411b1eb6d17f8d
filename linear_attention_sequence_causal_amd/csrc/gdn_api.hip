// gdn_api.hip -- C ABI of the gfx950 Gated DeltaNet mixer (see include/gdn.h).
//
// Host side only: argument validation (all before any HIP call), device
// check, workspace sizing and kernel launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/gdn.h"
#include "gdn_attention.h"
#include "gdn_device.h"
#include "gdn_linear.h"
#include "gdn_prefill_plan.h"

namespace gdn {
template <typename T>
hipError_t launch_decode(const void *q, const void *k, const void *v, const float *a,
                         const float *b, const void *z, const float *conv_w, const float *A_log,
                         const float *dt_bias, const float *norm_w, float q_scale, float l2_eps,
                         float rms_eps, void *state, int state_kind, float *state_scale,
                         void *conv_state, void *o, int batch, int Hk, int Hv, int gate,
                         hipStream_t stream);
int decode_max_ratio();
template <typename T>
hipError_t launch_decode_tokens(const void *q, const void *k, const void *v, const float *a,
                                const float *b, const void *z, const float *conv_w,
                                const float *A_log, const float *dt_bias, const float *norm_w,
                                float q_scale, float l2_eps, float rms_eps, float *state,
                                void *conv_state, const int32_t *num_commit, void *o, int batch,
                                int n, int Hk, int Hv, int gate, hipStream_t stream);
int decode_max_tokens();
}  // namespace gdn

namespace {

thread_local char g_err[512] = "";
thread_local gdn::PrefillTiming g_timing;

gdn_status fail(gdn_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

gdn_status hip_fail(hipError_t e, const char *what) {
  return fail(GDN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Per-device check that the current device is a gfx950, cached.
std::mutex g_dev_mu;
std::vector<int> g_dev_ok;  // -1 unknown, 0 no, 1 yes

gdn_status check_device() {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    return fail(GDN_ERR_NO_DEVICE, "no HIP device visible");
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(GDN_ERR_NO_DEVICE, "hipGetDevice failed");
  }
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if ((int)g_dev_ok.size() < count) g_dev_ok.resize(count, -1);
  if (g_dev_ok[dev] < 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return fail(GDN_ERR_NO_DEVICE, "hipGetDeviceProperties failed");
    }
    g_dev_ok[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
  }
  if (!g_dev_ok[dev]) return fail(GDN_ERR_NO_DEVICE, "device %d is not a gfx950", dev);
  return GDN_OK;
}

gdn_status check_params(const gdn_params *p) {
  if (!p) return fail(GDN_ERR_INVALID_ARGUMENT, "params is NULL");
  if (p->num_qk_heads <= 0 || p->num_v_heads <= 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "head counts must be positive (Hk=%d, Hv=%d)",
                p->num_qk_heads, p->num_v_heads);
  if (p->num_v_heads % p->num_qk_heads != 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "num_v_heads (%d) must be a multiple of num_qk_heads (%d)",
                p->num_v_heads, p->num_qk_heads);
  if (p->head_dim <= 0) return fail(GDN_ERR_INVALID_ARGUMENT, "head_dim must be positive");
  if (p->head_dim != gdn::kD)
    return fail(GDN_ERR_UNSUPPORTED, "head_dim %d: kernels are built for head_dim %d",
                p->head_dim, gdn::kD);
  if (p->act_dtype != GDN_BF16 && p->act_dtype != GDN_F32)
    return fail(GDN_ERR_INVALID_ARGUMENT, "act_dtype %d is not GDN_BF16 or GDN_F32", p->act_dtype);
  if (!p->conv_weight || !p->A_log || !p->dt_bias)
    return fail(GDN_ERR_INVALID_ARGUMENT, "conv_weight, A_log and dt_bias are required");
  if (!(p->l2_eps >= 0.0f) || !(p->rms_eps >= 0.0f))
    return fail(GDN_ERR_INVALID_ARGUMENT, "eps values must be >= 0");
  if (p->output_gate != GDN_GATE_SILU && p->output_gate != GDN_GATE_SIGMOID)
    return fail(GDN_ERR_INVALID_ARGUMENT, "output_gate %d is not GDN_GATE_SILU or GDN_GATE_SIGMOID",
                p->output_gate);
  return GDN_OK;
}

}  // namespace

extern "C" {

const char *gdn_status_string(gdn_status s) {
  switch (s) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_INVALID_ARGUMENT: return "GDN_ERR_INVALID_ARGUMENT";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE";
    case GDN_ERR_NO_DEVICE: return "GDN_ERR_NO_DEVICE";
    case GDN_ERR_HIP: return "GDN_ERR_HIP";
  }
  return "GDN_ERR_UNKNOWN";
}

const char *gdn_last_error(void) { return g_err; }

int gdn_prefill_last_kernel_times(float *ms, int max_kernels) {
  if (!g_timing.created || !g_timing.valid || !ms || max_kernels <= 0) return -1;
  if (hipEventSynchronize(g_timing.ev[gdn::kTimedKernels]) != hipSuccess) return -1;
  const int n = max_kernels < gdn::kTimedKernels ? max_kernels : gdn::kTimedKernels;
  for (int i = 0; i < n; ++i) {
    float t = 0.f;
    if (g_timing.ran[i] && hipEventElapsedTime(&t, g_timing.ev[i], g_timing.ev[i + 1]) != hipSuccess)
      t = 0.f;
    ms[i] = g_timing.ran[i] ? t : 0.f;
  }
  return n;
}

const char *gdn_version(void) { return "gdn-gfx950 0.2"; }

gdn_status gdn_check_device_errors(void *stream) {
  g_err[0] = 0;
  gdn_status st = check_device();
  if (st != GDN_OK) return st;
  if (hipError_t e = hipStreamSynchronize((hipStream_t)stream); e != hipSuccess)
    return hip_fail(e, "stream synchronisation");
  int flag = 0, aflag = 0;
  if (hipError_t e = gdn::take_prefill_error(&flag); e != hipSuccess)
    return hip_fail(e, "reading the device error flag");
  if (hipError_t e = gdn::take_attention_error(&aflag); e != hipSuccess)
    return hip_fail(e, "reading the attention error flag");
  if (flag)
    return fail(GDN_ERR_INVALID_ARGUMENT,
                "a gdn_prefill call on this device had invalid cu_seqlens contents (its o and "
                "final states were not written)");
  if (aflag)
    return fail(GDN_ERR_INVALID_ARGUMENT,
                "a gdn_gated_attention call on this device had invalid cu_seqlens contents "
                "(its o was not written)");
  return GDN_OK;
}

size_t gdn_prefill_workspace_bytes(const gdn_params *p, int32_t num_seqs, int64_t total_tokens) {
  if (check_params(p) != GDN_OK || num_seqs < 0 || total_tokens < 0) return (size_t)-1;
  gdn::PrefillPlan plan = gdn::make_plan(num_seqs, total_tokens, p->num_v_heads);
  return plan.workspace_bytes;
}

}  // extern "C"

namespace {
// noalloc: the workspace is the library's static device array (gdn_prefill_noalloc);
// then nothing here allocates or synchronises (GDN_VALIDATE and GDN_KERNEL_TIMING,
// which need host copies and events, are ignored).
gdn_status prefill_impl(const void *q, const void *k, const void *v, const float *a,
                        const float *b, const void *z, const gdn_params *p,
                        const float *init_state, const int32_t *cu_seqlens, int32_t num_seqs,
                        int64_t total_tokens, const void *conv_state_in, void *o,
                        float *final_state, void *conv_state_out, void *workspace,
                        size_t workspace_bytes, void *stream, bool noalloc) {
  g_err[0] = 0;
  gdn_status st = check_params(p);
  if (st != GDN_OK) return st;
  if (num_seqs < 0 || total_tokens < 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "num_seqs (%d) and total_tokens (%lld) must be >= 0",
                num_seqs, (long long)total_tokens);
  if (total_tokens > 0 && (!q || !k || !v || !a || !b || !z || !o))
    return fail(GDN_ERR_INVALID_ARGUMENT, "q, k, v, a, b, z and o are required when T > 0");
  if (num_seqs > 0 && !final_state)
    return fail(GDN_ERR_INVALID_ARGUMENT, "final_state is required");
  if (!cu_seqlens && num_seqs != 1)
    return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens may be NULL only when num_seqs == 1");
  if (total_tokens > (int64_t)INT32_MAX)
    return fail(GDN_ERR_UNSUPPORTED, "total_tokens above 2^31-1");
  if (o && (o == q || o == k || o == v || o == z))
    return fail(GDN_ERR_INVALID_ARGUMENT, "o must not alias an input");
  gdn::PrefillPlan plan = gdn::make_plan(num_seqs, total_tokens, p->num_v_heads);
  if (noalloc) {
    if (plan.workspace_bytes > gdn::kStaticWorkspaceBytes)
      return fail(GDN_ERR_WORKSPACE,
                  "this problem needs %zu bytes of workspace; gdn_prefill_noalloc has %zu",
                  plan.workspace_bytes, gdn::kStaticWorkspaceBytes);
  } else {
    if (plan.workspace_bytes > 0 && (!workspace || workspace_bytes < plan.workspace_bytes))
      return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given",
                  plan.workspace_bytes, workspace ? workspace_bytes : (size_t)0);
    if (workspace && ((uintptr_t)workspace & 255u))
      return fail(GDN_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  }
  st = check_device();
  if (st != GDN_OK) return st;
  if (noalloc) {
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (hipError_t e = gdn::static_workspace(dev, &workspace); e != hipSuccess)
      return hip_fail(e, "address of the static workspace");
  }
  if (num_seqs == 0) return GDN_OK;

  const char *validate = noalloc ? nullptr : getenv("GDN_VALIDATE");
  if (validate && validate[0] == '1') {
    // report an invalid table met by an earlier call first
    if (hipError_t e = hipStreamSynchronize((hipStream_t)stream); e != hipSuccess)
      return hip_fail(e, "GDN_VALIDATE stream synchronisation");
    int flag = 0;
    if (hipError_t e = gdn::take_prefill_error(&flag); e != hipSuccess)
      return hip_fail(e, "GDN_VALIDATE error flag");
    if (flag)
      return fail(GDN_ERR_INVALID_ARGUMENT,
                  "an earlier gdn_prefill call on this device had invalid cu_seqlens");
  }
  if (validate && validate[0] == '1' && cu_seqlens) {
    std::vector<int32_t> cu(num_seqs + 1);
    hipError_t e = hipMemcpy(cu.data(), cu_seqlens, sizeof(int32_t) * (num_seqs + 1),
                             hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "GDN_VALIDATE copy of cu_seqlens");
    if (cu[0] != 0) return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens[0] = %d, expected 0", cu[0]);
    for (int i = 0; i < num_seqs; ++i)
      if (cu[i + 1] < cu[i])
        return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens decreases at %d", i);
    if (cu[num_seqs] != total_tokens)
      return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens[N] = %d, expected total_tokens %lld",
                  cu[num_seqs], (long long)total_tokens);
  }
  gdn::PrefillTiming *tm = nullptr;
  const char *tv = noalloc ? nullptr : getenv("GDN_KERNEL_TIMING");
  if (tv && tv[0] == '1') {
    if (!g_timing.created) {
      for (int i = 0; i <= gdn::kTimedKernels; ++i) {
        hipError_t ce = hipEventCreate(&g_timing.ev[i]);
        if (ce != hipSuccess) return hip_fail(ce, "hipEventCreate");
      }
      g_timing.created = true;
    }
    tm = &g_timing;
  }
  hipError_t e = gdn::launch_prefill(plan, q, k, v, a, b, z, *p, init_state, cu_seqlens,
                                     num_seqs, total_tokens, conv_state_in, o, final_state,
                                     conv_state_out, workspace, (hipStream_t)stream, tm);
  if (tm) tm->valid = (e == hipSuccess);
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return GDN_OK;
}
}  // namespace

extern "C" {

gdn_status gdn_prefill(const void *q, const void *k, const void *v, const float *a, const float *b,
                       const void *z, const gdn_params *p, const float *init_state,
                       const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                       const void *conv_state_in, void *o, float *final_state,
                       void *conv_state_out, void *workspace, size_t workspace_bytes,
                       void *stream) {
  return prefill_impl(q, k, v, a, b, z, p, init_state, cu_seqlens, num_seqs, total_tokens,
                      conv_state_in, o, final_state, conv_state_out, workspace, workspace_bytes,
                      stream, false);
}

gdn_status gdn_prefill_noalloc(const void *q, const void *k, const void *v, const float *a,
                               const float *b, const void *z, const gdn_params *p,
                               const float *init_state, const int32_t *cu_seqlens,
                               int32_t num_seqs, int64_t total_tokens, const void *conv_state_in,
                               void *o, float *final_state, void *conv_state_out, void *stream) {
  return prefill_impl(q, k, v, a, b, z, p, init_state, cu_seqlens, num_seqs, total_tokens,
                      conv_state_in, o, final_state, conv_state_out, nullptr, 0, stream, true);
}

}  // extern "C"

namespace {
// state_kind: 0 fp32, 1 bf16, 2 fp8 (E4M3 values + per-row scales in state_scale)
gdn_status decode_step_impl(const void *q, const void *k, const void *v, const float *a,
                            const float *b, const void *z, const gdn_params *p, void *state,
                            int state_kind, float *state_scale, void *conv_state, void *o,
                            int32_t batch, void *stream) {
  g_err[0] = 0;
  gdn_status st = check_params(p);
  if (st != GDN_OK) return st;
  if (batch < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "batch (%d) must be >= 0", batch);
  if (p->num_v_heads / p->num_qk_heads > gdn::decode_max_ratio())
    return fail(GDN_ERR_UNSUPPORTED, "num_v_heads / num_qk_heads above %d",
                gdn::decode_max_ratio());
  if (batch > 0 && (!q || !k || !v || !a || !b || !z || !state || !conv_state || !o))
    return fail(GDN_ERR_INVALID_ARGUMENT, "all tensor pointers are required");
  if (batch > 0 && state_kind == 2 && !state_scale)
    return fail(GDN_ERR_INVALID_ARGUMENT, "state_scale is required with fp8 state storage");
  if ((int64_t)batch * p->num_qk_heads > (int64_t)INT32_MAX)
    return fail(GDN_ERR_UNSUPPORTED, "batch * num_qk_heads too large");
  if (o && (o == q || o == k || o == v || o == z))
    return fail(GDN_ERR_INVALID_ARGUMENT, "o must not alias an input");
  st = check_device();
  if (st != GDN_OK) return st;
  hipError_t e;
  if (p->act_dtype == GDN_BF16)
    e = gdn::launch_decode<gdn::bf16_t>(q, k, v, a, b, z, p->conv_weight, p->A_log, p->dt_bias,
                                        p->norm_weight, p->q_scale, p->l2_eps, p->rms_eps, state,
                                        state_kind, state_scale, conv_state, o, batch,
                                        p->num_qk_heads, p->num_v_heads, p->output_gate,
                                        (hipStream_t)stream);
  else
    e = gdn::launch_decode<float>(q, k, v, a, b, z, p->conv_weight, p->A_log, p->dt_bias,
                                  p->norm_weight, p->q_scale, p->l2_eps, p->rms_eps, state,
                                  state_kind, state_scale, conv_state, o, batch, p->num_qk_heads,
                                  p->num_v_heads, p->output_gate, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return GDN_OK;
}
}  // namespace

extern "C" {

gdn_status gdn_decode_step(const void *q, const void *k, const void *v, const float *a,
                           const float *b, const void *z, const gdn_params *p, float *state,
                           void *conv_state, void *o, int32_t batch, void *stream) {
  return decode_step_impl(q, k, v, a, b, z, p, state, 0, nullptr, conv_state, o, batch, stream);
}

gdn_status gdn_decode_step_bf16_state(const void *q, const void *k, const void *v,
                                      const float *a, const float *b, const void *z,
                                      const gdn_params *p, void *state, void *conv_state,
                                      void *o, int32_t batch, void *stream) {
  return decode_step_impl(q, k, v, a, b, z, p, state, 1, nullptr, conv_state, o, batch, stream);
}

gdn_status gdn_decode_step_fp8_state(const void *q, const void *k, const void *v,
                                     const float *a, const float *b, const void *z,
                                     const gdn_params *p, void *state, float *state_scale,
                                     void *conv_state, void *o, int32_t batch, void *stream) {
  return decode_step_impl(q, k, v, a, b, z, p, state, 2, state_scale, conv_state, o, batch,
                          stream);
}

gdn_status gdn_decode_tokens(const void *q, const void *k, const void *v, const float *a,
                             const float *b, const void *z, const gdn_params *p, float *state,
                             void *conv_state, const int32_t *num_commit, void *o, int32_t batch,
                             int32_t n_tokens, void *stream) {
  g_err[0] = 0;
  gdn_status st = check_params(p);
  if (st != GDN_OK) return st;
  if (batch < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "batch (%d) must be >= 0", batch);
  if (n_tokens < 1 || n_tokens > gdn::decode_max_tokens())
    return fail(GDN_ERR_INVALID_ARGUMENT, "n_tokens (%d) must be in 1..%d", n_tokens,
                gdn::decode_max_tokens());
  if (p->num_v_heads / p->num_qk_heads > gdn::decode_max_ratio())
    return fail(GDN_ERR_UNSUPPORTED, "num_v_heads / num_qk_heads above %d",
                gdn::decode_max_ratio());
  if (batch > 0 && (!q || !k || !v || !a || !b || !z || !state || !conv_state || !o))
    return fail(GDN_ERR_INVALID_ARGUMENT, "all tensor pointers except num_commit are required");
  if ((int64_t)batch * p->num_qk_heads > (int64_t)INT32_MAX)
    return fail(GDN_ERR_UNSUPPORTED, "batch * num_qk_heads too large");
  if (o && (o == q || o == k || o == v || o == z))
    return fail(GDN_ERR_INVALID_ARGUMENT, "o must not alias an input");
  st = check_device();
  if (st != GDN_OK) return st;
  hipError_t e;
  if (p->act_dtype == GDN_BF16)
    e = gdn::launch_decode_tokens<gdn::bf16_t>(
        q, k, v, a, b, z, p->conv_weight, p->A_log, p->dt_bias, p->norm_weight, p->q_scale,
        p->l2_eps, p->rms_eps, state, conv_state, num_commit, o, batch, n_tokens,
        p->num_qk_heads, p->num_v_heads, p->output_gate, (hipStream_t)stream);
  else
    e = gdn::launch_decode_tokens<float>(
        q, k, v, a, b, z, p->conv_weight, p->A_log, p->dt_bias, p->norm_weight, p->q_scale,
        p->l2_eps, p->rms_eps, state, conv_state, num_commit, o, batch, n_tokens,
        p->num_qk_heads, p->num_v_heads, p->output_gate, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "decode_tokens launch");
  return GDN_OK;
}

}  // extern "C"

// ------------------------------------------------------------------ projections
namespace {
gdn_status linear_checks(const void *x, const void *w, int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N <= 0 || K <= 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "sizes must be M >= 0, N > 0, K > 0");
  if (M > 0 && (!x || !w)) return fail(GDN_ERR_INVALID_ARGUMENT, "x and w are required");
  if (K % gdn::kLinearKStep != 0)
    return fail(GDN_ERR_UNSUPPORTED, "K (%lld) must be a multiple of %d", (long long)K,
                gdn::kLinearKStep);
  if (N > (int64_t)INT32_MAX || K > (int64_t)INT32_MAX / 256)
    return fail(GDN_ERR_UNSUPPORTED, "N or K too large");
  return GDN_OK;
}
// The projections read only the head layout and the activation dtype of p.
gdn_status check_layout(const gdn_params *p) {
  if (!p) return fail(GDN_ERR_INVALID_ARGUMENT, "params is NULL");
  if (p->num_qk_heads <= 0 || p->num_v_heads <= 0 || p->num_v_heads % p->num_qk_heads != 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "head counts must be positive, Hv a multiple of Hk");
  if (p->head_dim <= 0) return fail(GDN_ERR_INVALID_ARGUMENT, "head_dim must be positive");
  if (p->act_dtype != GDN_BF16 && p->act_dtype != GDN_F32)
    return fail(GDN_ERR_INVALID_ARGUMENT, "act_dtype %d is not GDN_BF16 or GDN_F32", p->act_dtype);
  return GDN_OK;
}
}  // namespace

extern "C" {

gdn_status gdn_linear(const void *x, const void *w, int64_t M, int32_t N, int32_t K, void *y,
                      void *stream) {
  g_err[0] = 0;
  gdn_status st = linear_checks(x, w, M, N, K);
  if (st != GDN_OK) return st;
  if (M > 0 && !y) return fail(GDN_ERR_INVALID_ARGUMENT, "y is required");
  if (M == 0) return GDN_OK;
  st = check_device();
  if (st != GDN_OK) return st;
  gdn::LinearOut out{};
  out.nseg = 1;
  out.ptr[0] = y;
  out.row_stride[0] = N;
  out.dtype[0] = gdn::kLinBf16;
  hipError_t e = gdn::launch_linear_bf16(x, w, M, N, K, out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "linear launch");
  return GDN_OK;
}

gdn_status gdn_in_projection(const void *x, const void *w_in, const gdn_params *p, int64_t T,
                             int32_t d_model, void *q, void *k, void *v, void *z, float *a,
                             float *b, void *stream) {
  g_err[0] = 0;
  gdn_status st = check_layout(p);
  if (st != GDN_OK) return st;
  const int64_t qk = (int64_t)p->num_qk_heads * p->head_dim, vd = (int64_t)p->num_v_heads * p->head_dim;
  const int64_t N = 2 * qk + 2 * vd + 2 * (int64_t)p->num_v_heads;
  st = linear_checks(x, w_in, T, N, d_model);
  if (st != GDN_OK) return st;
  if (T > 0 && (!q || !k || !v || !z || !a || !b))
    return fail(GDN_ERR_INVALID_ARGUMENT, "q, k, v, z, a and b are required");
  if (T == 0) return GDN_OK;
  st = check_device();
  if (st != GDN_OK) return st;
  const int act = p->act_dtype == GDN_BF16 ? gdn::kLinBf16 : gdn::kLinF32;
  gdn::LinearOut out{};
  out.nseg = 6;
  const int64_t begin[6] = {0, qk, 2 * qk, 2 * qk + vd, 2 * qk + 2 * vd,
                            2 * qk + 2 * vd + p->num_v_heads};
  void *ptrs[6] = {q, k, v, z, a, b};
  const int64_t strides[6] = {qk, qk, vd, vd, p->num_v_heads, p->num_v_heads};
  const int types[6] = {act, act, act, act, gdn::kLinF32, gdn::kLinF32};
  for (int i = 0; i < 6; ++i) {
    out.col_begin[i] = (int)begin[i];
    out.ptr[i] = ptrs[i];
    out.row_stride[i] = strides[i];
    out.dtype[i] = types[i];
  }
  hipError_t e = gdn::launch_linear_bf16(x, w_in, T, (int)N, d_model, out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "in-projection launch");
  return GDN_OK;
}

gdn_status gdn_out_projection(const void *o, const void *w_out, const gdn_params *p, int64_t T,
                              int32_t d_model, void *y, void *stream) {
  g_err[0] = 0;
  gdn_status st = check_layout(p);
  if (st != GDN_OK) return st;
  if (p->act_dtype != GDN_BF16)
    return fail(GDN_ERR_UNSUPPORTED, "the output projection takes bf16 o (act_dtype GDN_BF16)");
  return gdn_linear(o, w_out, T, d_model, p->num_v_heads * p->head_dim, y, stream);
}

}  // extern "C"

// ------------------------------------------------------------------ gated attention
namespace {
gdn_status check_attn(const gdn_attn_params *p, int64_t T) {
  if (!p) return fail(GDN_ERR_INVALID_ARGUMENT, "params is NULL");
  if (p->num_kv_heads <= 0 || p->num_q_heads <= 0 || p->num_q_heads % p->num_kv_heads != 0)
    return fail(GDN_ERR_INVALID_ARGUMENT,
                "head counts must be positive, num_q_heads (%d) a multiple of num_kv_heads (%d)",
                p->num_q_heads, p->num_kv_heads);
  if (p->head_dim <= 0) return fail(GDN_ERR_INVALID_ARGUMENT, "head_dim must be positive");
  if (p->head_dim != gdn::kAttnHeadDim)
    return fail(GDN_ERR_UNSUPPORTED, "head_dim %d: the attention kernels are built for %d",
                p->head_dim, gdn::kAttnHeadDim);
  if (p->rotary_dim < 0 || p->rotary_dim > p->head_dim || p->rotary_dim % 16 != 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "rotary_dim %d must be a multiple of 16 in [0, %d]",
                p->rotary_dim, p->head_dim);
  if (!(p->rope_theta > 0.f) || !(p->norm_eps >= 0.f))
    return fail(GDN_ERR_INVALID_ARGUMENT, "rope_theta must be > 0 and norm_eps >= 0");
  if (T < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "total_tokens must be >= 0");
  if (T * (int64_t)(p->num_q_heads + p->num_kv_heads) >= ((int64_t)1 << 27))
    return fail(GDN_ERR_UNSUPPORTED, "total_tokens * (Hq + Hkv) must be below 2^27");
  return GDN_OK;
}
}  // namespace

extern "C" {

size_t gdn_gated_attention_workspace_bytes(const gdn_attn_params *p, int64_t total_tokens) {
  if (check_attn(p, total_tokens) != GDN_OK) return (size_t)-1;
  return gdn::attention_workspace_bytes(total_tokens, p->num_q_heads, p->num_kv_heads);
}

gdn_status gdn_gated_attention(const void *q, const void *k, const void *v, const void *gate,
                               const gdn_attn_params *p, const int32_t *cu_seqlens,
                               int32_t num_seqs, int64_t total_tokens, void *o,
                               void *workspace, size_t workspace_bytes, void *stream) {
  g_err[0] = 0;
  gdn_status st = check_attn(p, total_tokens);
  if (st != GDN_OK) return st;
  const int64_t T = total_tokens;
  if (num_seqs < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "num_seqs must be >= 0");
  if (num_seqs == 0 && T != 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "total_tokens must be 0 when num_seqs is 0");
  if (!cu_seqlens && num_seqs != 1)
    return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens may be NULL only when num_seqs == 1");
  if (T > 0 && (!q || !k || !v || !gate || !o))
    return fail(GDN_ERR_INVALID_ARGUMENT, "q, k, v, gate and o are required when T > 0");
  if (o && (o == q || o == k || o == v || o == gate))
    return fail(GDN_ERR_INVALID_ARGUMENT, "o must not alias an input");
  const size_t need = gdn::attention_workspace_bytes(T, p->num_q_heads, p->num_kv_heads);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (workspace && ((uintptr_t)workspace & 255u))
    return fail(GDN_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  st = check_device();
  if (st != GDN_OK) return st;
  if (T == 0) return GDN_OK;
  const char *validate = getenv("GDN_VALIDATE");
  if (validate && validate[0] == '1' && cu_seqlens) {
    std::vector<int32_t> cu(num_seqs + 1);
    hipError_t e = hipMemcpy(cu.data(), cu_seqlens, sizeof(int32_t) * (num_seqs + 1),
                             hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "GDN_VALIDATE copy of cu_seqlens");
    if (cu[0] != 0) return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens[0] = %d, expected 0", cu[0]);
    for (int i = 0; i < num_seqs; ++i)
      if (cu[i + 1] < cu[i])
        return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens decreases at %d", i);
    if (cu[num_seqs] != T)
      return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens[N] = %d, expected total_tokens %lld",
                  cu[num_seqs], (long long)T);
  }
  const float scale = p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)p->head_dim);
  hipError_t e = gdn::launch_attention(q, k, v, gate, cu_seqlens, num_seqs, T, p->num_q_heads,
                                       p->num_kv_heads, p->q_norm_weight, p->k_norm_weight,
                                       p->rotary_dim, p->rope_theta, p->norm_eps, scale,
                                       workspace, o, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "gated attention launch");
  return GDN_OK;
}

}  // extern "C"
