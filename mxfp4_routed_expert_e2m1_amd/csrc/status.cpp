// status.cpp -- status strings and the cached per-device queries.
#include <hip/hip_runtime.h>
#include <string.h>

#include "../../include/moe_mxfp4.h"

namespace moe {

// -1 unknown, 0 no, 1 yes; indexed by device ordinal.
static int g_arch_ok[64] = {
    -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1,
    -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1,
    -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1};

bool device_is_gfx950() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return false;
  if (dev < 64 && g_arch_ok[dev] >= 0) return g_arch_ok[dev] == 1;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return false;
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) g_arch_ok[dev] = ok ? 1 : 0;
  return ok;
}

// Compute units of the current device (0 if unknown), cached per device.
static int g_cus[64] = {0};

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && g_cus[dev] > 0) return g_cus[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) g_cus[dev] = n;
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
