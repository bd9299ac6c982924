// Helpers of the C-ABI layer shared between its source files (internal to
// libssd_mi355x.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "ssd.h"

namespace ssd {

// Status of `dims` as ssd_forward checks it (host only, no HIP call); when
// SSD_OK, *ws_bytes receives ssd_forward_workspace_bytes(dims).
ssd_status forward_dims_check(const ssd_dims *dims, size_t *ws_bytes);

// SSD_OK for hipSuccess; otherwise records e as the calling thread's last
// HIP error (ssd_last_hip_error) and returns SSD_ERR_HIP.
ssd_status hip_error(hipError_t e);

}  // namespace ssd
