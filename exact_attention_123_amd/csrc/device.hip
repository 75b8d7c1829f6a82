// Host-side queries of the current HIP device (see device.h).  Each device's
// architecture check and compute-unit count are read with one
// hipGetDeviceProperties call, the first time an entry point runs on it, and
// kept in per-device atomics (entry points may be called from several host
// threads).

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "device.h"

namespace attn_internal {

namespace {

constexpr int kMaxDevices = 64;
// per device: 0 not read yet, 1 a gfx950, 2 another device
std::atomic<int> g_arch[kMaxDevices];
std::atomic<int> g_cus[kMaxDevices];

// The current device's index, or -1.
int current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
  return dev;
}

// Reads and caches the device's properties; returns its architecture state.
int arch_state(int dev) {
  int s = g_arch[dev].load(std::memory_order_relaxed);
  if (s == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 2;
    s = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    g_arch[dev].store(s, std::memory_order_relaxed);
  }
  return s;
}

}  // namespace

attn_status check_device() {
  const int dev = current_device();
  if (dev < 0) return ATTN_ERR_DEVICE;
  return arch_state(dev) == 1 ? ATTN_OK : ATTN_ERR_DEVICE;
}

int device_cus() {
  const int dev = current_device();
  if (dev < 0 || arch_state(dev) != 1) return 256;
  const int n = g_cus[dev].load(std::memory_order_relaxed);
  return n > 0 ? n : 256;
}

}  // namespace attn_internal
