// Per-device facts the launchers need, queried once per device.  The caches
// are atomics: concurrent first calls may both query the runtime, and both
// store the same value.
#include <atomic>

#include "dit_internal.h"

namespace dit {

hipError_t current_device(int* dev) {
  hipError_t e = hipGetDevice(dev);
  if (e != hipSuccess) return e;
  if (*dev < 0 || *dev >= kMaxDevices) return hipErrorInvalidDevice;
  return hipSuccess;
}

hipError_t device_cu_count(int* cus) {
  static std::atomic<int> cached[kMaxDevices];  // zero-initialised (static storage)
  int dev = 0;
  hipError_t e = current_device(&dev);
  if (e != hipSuccess) return e;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (n < 1) n = 1;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  *cus = n;
  return hipSuccess;
}

}  // namespace dit
