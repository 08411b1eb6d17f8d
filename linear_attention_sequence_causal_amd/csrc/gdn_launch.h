// gdn_launch.h -- host helpers shared by the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

namespace gdn {

// Raises a kernel's dynamic LDS limit to `bytes` on the current device.  The attribute
// belongs to the device, so each device is set once (tracked in `done`, one bit per
// device id below 64; higher ids are set on every call).
inline hipError_t ensure_lds_limit(const void *fn, int bytes, std::atomic<uint64_t> &done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t)1 << dev : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}

}  // namespace gdn
