// Shared-prefix groups for single-token decode: host side (sizes, layout,
// applicability).  The device code is in pkv_group.h; detection runs in the
// planning kernel and the group items run on extra workgroups of the decode
// launch.  Also the cached device attributes and switches the launchers use.
#include <cstdlib>
#include <mutex>

#include "pkv_internal.h"

namespace pkv {

bool groups_enabled() {
  const char* v = std::getenv("PKV_PREFIX_GROUPS");
  return v && v[0] == '1';
}

int decode_tile_mode() {
  const char* v = std::getenv("PKV_DECODE_TILE");
  if (!v || !v[0]) return -1;
  return v[0] == '0' ? 0 : 1;
}

bool groups_supported(const DecodeArgs& a) {
  const int G = a.Hq / a.Hkv;
  // four waves per decode workgroup (Hq >= 16) so that group workgroups match
  // them; detection inside the single planning workgroup (B <= kGroupMaxB)
  return a.bf16 && a.T == 1 && a.B >= 2 && a.B <= kGroupMaxB && (a.D == 64 || a.D == 128) && G <= 32 &&
         a.Hq >= 16;
}

size_t group_workspace_bytes(int B, int Hq, int D) {
  const size_t r = 256;
  size_t off = 0;
  off += ((size_t)B * 4 + r - 1) / r * r * 2;                         // sfx, nch
  off += ((size_t)B * 16 + r - 1) / r * r;                            // desc
  off += ((size_t)B * kGroupChunks / 2 * 4 + r - 1) / r * r;          // clist
  off += (size_t)B * kGroupChunks * Hq * (D + 1) * 4;                 // partials
  return off;
}

GroupPlan group_plan_layout(void* base, int B, int Hq, int D) {
  const size_t r = 256;
  unsigned char* p = static_cast<unsigned char*>(base);
  GroupPlan gp{};
  const size_t vec = ((size_t)B * 4 + r - 1) / r * r;
  gp.sfx = reinterpret_cast<int*>(p); p += vec;
  gp.nch = reinterpret_cast<int*>(p); p += vec;
  gp.desc = reinterpret_cast<int4*>(p); p += ((size_t)B * 16 + r - 1) / r * r;
  gp.clist = reinterpret_cast<int*>(p); p += ((size_t)B * kGroupChunks / 2 * 4 + r - 1) / r * r;
  gp.part = reinterpret_cast<float*>(p);
  (void)Hq; (void)D;
  return gp;
}

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

bool inline_plan_enabled() {
  const char* v = std::getenv("PKV_INLINE_PLAN");
  return !(v && v[0] == '0');
}

}  // namespace pkv
