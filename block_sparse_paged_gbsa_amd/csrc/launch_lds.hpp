// Host-side launch helper for the kernels that size their dynamic LDS at run time.
#pragma once

#include <atomic>

#include <hip/hip_runtime.h>

namespace gbsa {

// Raise a kernel's dynamic-LDS limit to `bytes` (if above the 64 KiB default) once per device
// and size, not on every launch: launches then make no host-side call that a HIP graph
// capture could reject. `set` holds the limit already granted on each device.
constexpr int kMaxDevices = 64;
inline hipError_t ensure_dynamic_lds(const void* fn, std::atomic<int>* set, size_t bytes) {
    if (bytes <= 64 * 1024) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool cached = dev >= 0 && dev < kMaxDevices;
    if (cached && set[dev].load(std::memory_order_relaxed) >= (int)bytes) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess && cached) set[dev].store((int)bytes, std::memory_order_relaxed);
    return e;
}

}  // namespace gbsa
