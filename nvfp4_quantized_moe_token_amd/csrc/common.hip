// Library-wide entry points (version, status strings) and the device check.
#include <string.h>

#include "common.hpp"

namespace nvfp4moe {

// 0 = unknown, 1 = gfx950, 2 = other.  Benign race: every writer stores the
// same answer.
static int g_arch_ok[64];

int check_arch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return NVFP4MOE_EARCH;
  if (dev >= 0 && dev < 64 && g_arch_ok[dev]) return g_arch_ok[dev] == 1 ? NVFP4MOE_OK : NVFP4MOE_EARCH;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return NVFP4MOE_EARCH;
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev >= 0 && dev < 64) g_arch_ok[dev] = ok ? 1 : 2;
  return ok ? NVFP4MOE_OK : NVFP4MOE_EARCH;
}

static int g_cu_count[64];

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < 64 && g_cu_count[dev] > 0) return g_cu_count[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
  if (dev >= 0 && dev < 64) g_cu_count[dev] = n;
  return n;
}

__global__ void fill_u32_kernel(uint32_t* p, uint32_t v, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

}  // namespace nvfp4moe

extern "C" int nvfp4moe_abi_version(void) { return NVFP4MOE_ABI_VERSION; }

extern "C" const char* nvfp4moe_status_string(int status) {
  switch (status) {
    case NVFP4MOE_OK: return "ok";
    case NVFP4MOE_EINVAL: return "invalid argument (NULL pointer, negative size or bad enum)";
    case NVFP4MOE_ESHAPE: return "unsupported shape or alignment";
    case NVFP4MOE_EARCH: return "current device is not gfx950";
    case NVFP4MOE_ELAUNCH: return "kernel launch failed";
    case NVFP4MOE_EWORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}
