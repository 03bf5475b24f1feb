// Internal helpers shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "q4gemv.h"

namespace q4 {

// Returns Q4_OK when the calling thread's current HIP device is a gfx950,
// else Q4_EDEVICE.  The answer is cached per device ordinal.
int check_device();

// Maps the error left by a launch to Q4_OK / Q4_ELAUNCH.
inline int launch_status() {
    return hipGetLastError() == hipSuccess ? Q4_OK : Q4_ELAUNCH;
}

inline bool aligned(const void *p, size_t a) {
    return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

constexpr int kWave = 64;

}  // namespace q4
