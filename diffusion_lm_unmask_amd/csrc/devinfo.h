// devinfo.h — the current device's compute-unit count, queried once per
// device and cached, for the launch-shape choices that depend on it.  The
// entry points ask before their first launch, so an error returns before
// anything is enqueued, and repeated calls make no device query.
#pragma once
#include <hip/hip_runtime.h>

#include <atomic>

#include "../../include/dlm.h"

namespace dlmh {

inline int cu_count(int* cus) {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DLM_ERR_HIP;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus = c;
      return DLM_OK;
    }
  }
  int c = 0;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      c <= 0)
    return DLM_ERR_HIP;
  if (dev >= 0 && dev < 64) cache[dev].store(c, std::memory_order_relaxed);
  *cus = c;
  return DLM_OK;
}

}  // namespace dlmh
