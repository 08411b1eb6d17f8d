// gdn_noalloc.hip -- the library-owned workspace of gdn_prefill_noalloc.
//
// Callers that cannot allocate device memory (code under HIP graph capture, serving
// loops, harnesses that forbid hipMalloc) get the prefill's workspace from this
// file-scope device array instead.  Each device that runs the library holds its own
// copy, allocated with the code object and kept until the process ends.  In host
// code the array's name is only a host-side stand-in: its device address is looked
// up with hipGetSymbolAddress once per device (with that device current) and only
// that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdn_prefill_plan.h"

namespace gdn {

static __device__ __align__(256) unsigned char scratch[kStaticWorkspaceBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch_ptr[kMaxDevices] = {};  // per-device address of scratch (no allocation)
}  // namespace

hipError_t static_workspace(int dev, void **out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace gdn
