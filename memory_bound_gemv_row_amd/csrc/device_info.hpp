// device_info.hpp -- the properties of the current HIP device that the
// launch plans read (compute units, LDS one workgroup may hold), looked up
// once per device and kept for the life of the process.  Shared by the
// GEMV, quantiser and softmax entry points.
#pragma once

#include "gemv.h"

#include <hip/hip_runtime.h>

#include <mutex>

namespace gemv_device {

struct Device {
    int cus;       // compute units
    int lds_max;   // bytes of LDS one workgroup may hold
};

constexpr int kMaxDevices = 64;

// Properties of the current device; GEMV_E_DEVICE when there is none or its
// attributes cannot be read.  Thread-safe; one cache for the whole library
// (an inline function's statics are shared by every translation unit).
inline int current(Device* out)
{
    static std::mutex mutex;
    static Device cache[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return GEMV_E_DEVICE;
    std::lock_guard<std::mutex> lock(mutex);
    if (cache[dev].cus == 0) {
        int n = 0, lds = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0 ||
            hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
            lds <= 0)
            return GEMV_E_DEVICE;
        cache[dev] = {n, lds};
    }
    *out = cache[dev];
    return GEMV_OK;
}

}  // namespace gemv_device
