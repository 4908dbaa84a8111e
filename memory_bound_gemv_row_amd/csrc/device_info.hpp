// device_info.hpp -- what every launch of the library reads about the
// device: the properties of the current HIP device that the launch plans
// use (compute units, LDS one workgroup may hold), looked up once per
// device and kept for the life of the process, and the bound on a launch's
// work-items.  Shared by the GEMV, quantiser and softmax entry points.
#pragma once

#include "gemv.h"

#include <hip/hip_runtime.h>

#include <atomic>
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
// attributes cannot be read.  One cache for the whole library (an inline
// function's statics are shared by every translation unit), filled on the
// first call on each device and lock-free: a call reads two atomics.  Two
// threads that both find a device's slot empty both query it and store the
// same values; a slot is complete once its CU count is non-zero (stored last,
// with release order).
inline int current(Device* out)
{
    struct Slot {
        std::atomic<int> cus{0};
        std::atomic<int> lds_max{0};
    };
    static Slot cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return GEMV_E_DEVICE;
    Slot& slot = cache[dev];
    int cus = slot.cus.load(std::memory_order_acquire);
    if (cus == 0) {
        int lds = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0 ||
            hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
            lds <= 0)
            return GEMV_E_DEVICE;
        slot.lds_max.store(lds, std::memory_order_relaxed);
        slot.cus.store(cus, std::memory_order_release);
    }
    *out = Device{cus, slot.lds_max.load(std::memory_order_relaxed)};
    return GEMV_OK;
}

}  // namespace gemv_device
