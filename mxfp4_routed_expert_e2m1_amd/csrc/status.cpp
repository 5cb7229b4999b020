// status.cpp -- status strings and the cached per-device queries.
#include <hip/hip_runtime.h>
#include <string.h>

#include <atomic>

#include "../../include/moe_mxfp4.h"

namespace moe {

// Per-device caches, indexed by device ordinal (< 64), shared by every host
// thread that calls the library: atomics, so concurrent first calls on one
// device race benignly (both store the same value).
// g_arch: 0 unknown, 1 not gfx950, 2 gfx950.  g_cus: 0 unknown, else the count.
static std::atomic<int> g_arch[64];
static std::atomic<int> g_cus[64];

bool device_is_gfx950() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return false;
  if (dev < 64) {
    const int c = g_arch[dev].load(std::memory_order_relaxed);
    if (c != 0) return c == 2;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return false;
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) g_arch[dev].store(ok ? 2 : 1, std::memory_order_relaxed);
  return ok;
}

// Compute units of the current device (0 if unknown), cached per device.
int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = g_cus[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64 && n > 0) g_cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace moe

extern "C" const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_SHAPE: return "unsupported shape";
    case MOE_ERR_STRIDE: return "leading dimension smaller than a row";
    case MOE_ERR_WORKSPACE: return "workspace or destination too small";
    case MOE_ERR_ALIGNMENT: return "misaligned pointer or stride";
    case MOE_ERR_UNSUPPORTED_ARCH: return "current device is not gfx950";
    case MOE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}
