// gdn_attention.h -- host interface of the gated full-attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

constexpr int kAttnHeadDim = 256;

size_t attention_workspace_bytes(int64_t T, int Hq, int Hkv);
// Reads, and clears, the flag an attention call with an invalid cu_seqlens table sets.
hipError_t take_attention_error(int *flag);
hipError_t launch_attention(const void *q, const void *k, const void *v, const void *gate,
                            const int32_t *cu, int N, int64_t T, int Hq, int Hkv,
                            const float *wq, const float *wk, int rotary_dim, float theta,
                            float eps, float scale, void *workspace, void *o,
                            hipStream_t stream);

}  // namespace gdn
