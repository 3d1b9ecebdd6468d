// Per-device runtime state of the library: the architecture check every
// entry point makes after its (HIP-free) argument validation.
//
// The kernels are built for gfx950 only.  A call on any other device would
// fail at launch with an opaque "no kernel image" error, so each entry point
// asks, before its first launch on a device, whether that device is a gfx950;
// the answer is cached per device, so later calls cost one hipGetDevice.
#include <hip/hip_runtime.h>

#include <atomic>

#include "ss_internal.h"

namespace ss {
namespace {

constexpr int kMaxDevices = 64;
// 0: not asked yet, 1: supported, 2: not a gfx950
std::atomic<int> g_arch_state[kMaxDevices];

}  // namespace

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return SS_ERR_HIP;
  if (dev >= kMaxDevices) return SS_ERR_UNSUPPORTED;
  int s = g_arch_state[dev].load(std::memory_order_acquire);
  if (s == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return SS_ERR_HIP;
    s = ss_scan_arch_supported(prop.gcnArchName) == SS_OK ? 1 : 2;
    g_arch_state[dev].store(s, std::memory_order_release);
  }
  return s == 1 ? SS_OK : SS_ERR_UNSUPPORTED;
}

}  // namespace ss
