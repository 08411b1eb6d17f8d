// gdn_prefill_plan.h -- launch plan of the chunked prefill (host side).
//
// Long sequences are cut into segments of `seg_len` tokens (a multiple of the
// 32-token chunk) so that several workgroups per v head run at once:
//   pass 1  (map):     per non-final segment s, the affine map of its chunks,
//                      H_end = A_s H_start + B_s  (A_s, B_s fp32 [D][D])
//   pass 2  (combine): per sequence, the start state of every segment,
//                      H_{s+1} = A_s H_s + B_s, sequential over segments; where
//                      A_s is zero (flagged by pass 1) H_{s+1} is B_s itself
//   pass 3  (full):    per segment, the chunk recurrence from its start state
//                      (the initial state, B_{s-1}, or what pass 2 wrote) with
//                      the fused prologue and epilogue; writes o and, for the
//                      last segment, the final state.
// A sequence that fits in one segment runs pass 3 only.  The segment table is
// built on the device from cu_seqlens, so the host needs only N and T; a call with
// one sequence builds none (each kernel forms the records it reads, and checks a
// given cu_seqlens itself).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/gdn.h"

namespace gdn {

// One segment of one sequence, built on the device from cu_seqlens.
struct SegInfo {
  int32_t seq;        // sequence index
  int32_t begin;      // first token (absolute, packed index)
  int32_t len;        // tokens in this segment (0 only for an empty sequence)
  int32_t idx;        // segment index within its sequence
  int32_t nseg;       // segments of its sequence
  int32_t first;      // global index of the sequence's first segment
  int32_t map;        // map slot if this is not the last segment, else -1
  int32_t seq_begin;  // first token of the sequence
};

struct PrefillPlan {
  int32_t num_seqs = 0;
  int64_t total_tokens = 0;
  int32_t num_v_heads = 0;
  int32_t seg_len = 0;       // tokens per segment (multiple of 32)
  int64_t max_segments = 0;  // upper bound of the segment count
  int64_t max_maps = 0;      // upper bound of the non-final segment count
  size_t off_table = 0, off_maps = 0, off_start = 0, off_flags = 0;
  size_t workspace_bytes = 0;
};

PrefillPlan make_plan(int32_t num_seqs, int64_t total_tokens, int32_t num_v_heads);

// Optional events between the prefill kernels (GDN_KERNEL_TIMING=1).
constexpr int kTimedKernels = 5;
struct PrefillTiming {
  hipEvent_t ev[kTimedKernels + 1];
  bool created = false, valid = false;
  bool ran[kTimedKernels];
};

// The static workspace of gdn_prefill_noalloc: one array of this many bytes per
// device (gdn_noalloc.hip), addressed through hipGetSymbolAddress on the device.
constexpr size_t kStaticWorkspaceBytes = (size_t)128 << 20;
// Device address of that array on device `dev` (the current device), looked up
// once per device and cached.
hipError_t static_workspace(int dev, void **out);

// Reads and clears this device's flag for invalid cu_seqlens contents (set by the
// segment table of an earlier gdn_prefill call).  Synchronous.
hipError_t take_prefill_error(int *flag);

hipError_t launch_prefill(const PrefillPlan &plan, const void *q, const void *k, const void *v,
                          const float *a, const float *b, const void *z, const gdn_params &p,
                          const float *init_state, const int32_t *cu_seqlens, int32_t num_seqs,
                          int64_t total_tokens, const void *conv_state_in, void *o,
                          float *final_state, void *conv_state_out, void *workspace,
                          hipStream_t stream, PrefillTiming *timing);

}  // namespace gdn
