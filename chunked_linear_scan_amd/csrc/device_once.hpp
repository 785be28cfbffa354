// One-time set-up per device (kernel attributes), safe to reach from several
// host threads at once.
#pragma once

#include <hip/hip_runtime.h>

#include <mutex>

namespace cls {

constexpr int kMaxDevices = 64;

// One per call site (a function-local static): a once flag and the status of
// the set-up for each device.
struct DeviceOnce {
    std::once_flag flag[kMaxDevices];
    int status[kMaxDevices] = {};
};

// Runs fn() (returning 0 or a negative status) once per device for `once`,
// on the first call made with that device current, and returns its status on
// every call.  Devices past kMaxDevices run fn() every time.
template <typename F>
int run_once_per_device(DeviceOnce& once, F&& fn) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return fn();
    std::call_once(once.flag[dev], [&] { once.status[dev] = fn(); });
    return once.status[dev];
}

}  // namespace cls
