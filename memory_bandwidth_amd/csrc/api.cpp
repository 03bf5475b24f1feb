// Library-wide entry points: status strings, ABI version, device check.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "q4_common.h"

namespace q4 {

namespace {
constexpr int kMaxDevices = 64;
// 0 = not yet checked, 1 = gfx950, 2 = unsupported.
std::atomic<int> g_device_state[kMaxDevices];
}  // namespace

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return Q4_EDEVICE;
    int st = g_device_state[dev].load(std::memory_order_acquire);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return Q4_EDEVICE;
        st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_device_state[dev].store(st, std::memory_order_release);
    }
    return st == 1 ? Q4_OK : Q4_EDEVICE;
}

}  // namespace q4

extern "C" const char *q4_strerror(int status) {
    switch (status) {
    case Q4_OK: return "ok";
    case Q4_EINVAL: return "invalid size, shape or group size";
    case Q4_ENULL: return "required pointer is NULL";
    case Q4_EALIGN: return "pointer breaks its alignment rule";
    case Q4_EDEVICE: return "no HIP device, or the current device is not gfx950";
    case Q4_ELAUNCH: return "kernel launch failed";
    default: return "unknown q4 status";
    }
}

extern "C" int q4_abi_version(void) { return Q4GEMV_ABI_VERSION; }
