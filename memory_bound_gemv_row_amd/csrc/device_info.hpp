// device_info.hpp -- what every launch of the library reads about the
// device: the properties of the current HIP device that the launch plans
// use (compute units, LDS one workgroup may hold), looked up once per
// device and kept for the life of the process, and the bound on a launch's
// work-items.  Shared by the GEMV, quantiser and softmax entry points.
#pragma once

#include "gemv.h"

#include <hip/hip_runtime.h>

#include <mutex>
#include <stdint.h>

namespace gemv_device {

struct Device {
    int cus;       // compute units
    int lds_max;   // bytes of LDS one workgroup may hold
};

constexpr int kMaxDevices = 64;

// A dispatch counts its work-items in 32 bits, so every launch keeps
// grid x block at or below 2^30; the kernels walk whatever rows (or row
// groups) lie beyond their grid.
constexpr int64_t kMaxWorkItems = int64_t(1) << 30;

inline int capped_grid(int64_t grid, int block)
{
    const int64_t cap = kMaxWorkItems / block;
    return (int)(grid < cap ? grid : cap);
}

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
