// Per-device runtime state of the library: the architecture check every
// entry point makes after its (HIP-free) argument validation, and the static
// scratch array of the non-allocating forward.
//
// The kernels are built for gfx950 only.  A call on any other device would
// fail at launch with an opaque "no kernel image" error, so each entry point
// asks, before its first launch on a device, whether that device is a gfx950;
// the answer is cached per device, so later calls cost one hipGetDevice.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "ss_internal.h"

namespace ss {
namespace {

constexpr int kMaxDevices = 64;
// 0: not asked yet, 1: supported, 2: not a gfx950
std::atomic<int> g_arch_state[kMaxDevices];

}  // namespace

// Scratch of ss_scan_fwd_noalloc (chunk carries, padded B/C rows): a static
// device array, so that the call needs no allocation.  Every GPU the library
// runs on holds its own copy until the process ends.  In host code the name
// `scratch` is only a host-side stand-in: its device address on the current
// GPU comes from hipGetSymbolAddress, looked up once per device.
static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

int static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return SS_ERR_HIP;
  if (dev >= kMaxDevices) return SS_ERR_UNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      // with the device current (hipGetDevice above): this GPU's copy of the array
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SS_ERR_HIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return SS_OK;
}

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
