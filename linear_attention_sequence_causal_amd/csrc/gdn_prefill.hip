// gdn_prefill.hip -- chunked prefill of the Gated DeltaNet mixer, gfx950 (in progress).
#include "gdn_device.h"
#include "gdn_prefill_plan.h"

namespace gdn {

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
                 sizeof(int32_t) * (size_t)p.max_maps);
  if (p.max_maps > 0) {
    p.off_maps = off;
    off = align256(off + 2 * DD * (size_t)p.max_maps * num_v_heads);
    p.off_start = off;
    off = align256(off + DD * (size_t)p.max_segments * num_v_heads);
  }
  p.workspace_bytes = off;
  return p;
}

hipError_t launch_prefill(const PrefillPlan &, const void *, const void *, const void *,
                          const float *, const float *, const void *, const gdn_params &,
                          const float *, const int32_t *, int32_t, int64_t, const void *, void *,
                          float *, void *, void *, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace gdn
