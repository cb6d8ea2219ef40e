// flint_common.h -- host helpers shared by the C-ABI source files: the
// last-HIP-error record and the device check.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flint {

// records e as the last HIP error and returns FLINT_E_HIP
int32_t api_hip_fail(hipError_t e);
// FLINT_OK when the current device is gfx950 (cached per device)
int32_t api_check_device();

}  // namespace flint
