// gdn_linear.h -- host interface of the MFMA linear layers (gdn_linear.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

constexpr int kMaxLinearSegs = 8;
constexpr int kLinBf16 = 0, kLinF32 = 1;
constexpr int kLinearKStep = 64;  // K must be a multiple of this

// Column ranges of C = A W^T and where they go: columns col_begin[s] .. col_begin[s+1]-1
// (the last one to N) are written to ptr[s] as rows of row_stride[s] elements of
// dtype[s], column col at ptr[s][row * row_stride[s] + col - col_begin[s]].
// col_begin[0] = 0, increasing.
struct LinearOut {
  int nseg;
  int col_begin[kMaxLinearSegs];
  void *ptr[kMaxLinearSegs];
  int64_t row_stride[kMaxLinearSegs];
  int dtype[kMaxLinearSegs];
};

size_t linear_lds_bytes();
hipError_t launch_linear_bf16(const void *A, const void *W, int64_t M, int N, int K,
                              const LinearOut &out, hipStream_t stream);

}  // namespace gdn
