// Device attributes the launchers size their grids and LDS by, read once per
// device and cached.
#include <mutex>

#include "pkv_internal.h"

namespace pkv {

namespace {
// A device attribute of the current device, cached per device; `fallback`
// when it cannot be read.
int cached_attribute(hipDeviceAttribute_t attr, int slot, int fallback) {
  constexpr int kMaxDevices = 64;
  static int vals[2][kMaxDevices];
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return fallback;
  std::lock_guard<std::mutex> lock(mu);
  if (vals[slot][dev] == 0) {
    int n = 0;
    vals[slot][dev] = hipDeviceGetAttribute(&n, attr, dev) == hipSuccess && n > 0 ? n : fallback;
  }
  return vals[slot][dev];
}
}  // namespace

int device_cus() { return cached_attribute(hipDeviceAttributeMultiprocessorCount, 0, 256); }

int device_lds_per_block() { return cached_attribute(hipDeviceAttributeMaxSharedMemoryPerBlock, 1, 65536); }

}  // namespace pkv
