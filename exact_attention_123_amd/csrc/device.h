// Host-side queries of the current HIP device, shared by the library's entry
// points (forward, backward, decode, materialised forward): whether it is a
// gfx950, and its compute-unit count, both read once per device and cached.
#ifndef ATTN_DEVICE_H_
#define ATTN_DEVICE_H_

#include "attn.h"

namespace attn_internal {

// ATTN_OK when the current device is an AMD gfx950 GPU, else ATTN_ERR_DEVICE
// (also when no device is current or its properties cannot be read).
attn_status check_device();

// Compute units of the current device; 256 (an MI355X's count) when no
// gfx950 device is current.  The kernels' launch plans compare grid sizes
// with it.
int device_cus();

}  // namespace attn_internal

#endif  // ATTN_DEVICE_H_
