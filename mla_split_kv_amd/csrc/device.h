// Device facts the launch plans need, shared by the library's sources.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>

namespace mla_dev {

// Compute units of the current device (256 on an MI355X), asked of the
// runtime once per device and cached; 256 if the runtime cannot tell.
inline int device_cus() {
  constexpr int MAX_DEVICES = 64;
  static std::atomic<int> cached[MAX_DEVICES];  // 0: not asked yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  const bool slot = dev >= 0 && dev < MAX_DEVICES;
  if (slot) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (slot) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

}  // namespace mla_dev
