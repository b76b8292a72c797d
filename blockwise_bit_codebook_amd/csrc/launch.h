// Host-side launch geometry shared by the HIP translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "device.h"
#include "kbit_internal.h"

namespace kbit {

// Resident workgroups per CU of `kern` launched with `threads` threads on
// the current device (with `dyn_lds` bytes of dynamic LDS per workgroup).
// Computed once per device and kept in `cache` (one
// slot per device ordinal, zero = not yet known); concurrent callers at
// worst compute the same value twice and store it with a relaxed atomic.
template <class Kern>
int cached_blocks_per_cu(Kern kern, int threads, std::atomic<int> (&cache)[kMaxDevices], size_t dyn_lds = 0) {
    const int dev = current_device_index();
    std::atomic<int>* slot = (dev >= 0 && dev < kMaxDevices) ? &cache[dev] : nullptr;
    int b = slot ? slot->load(std::memory_order_relaxed) : 0;
    if (b == 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, kern, threads, dyn_lds) != hipSuccess || b < 1) b = 1;
        if (slot) slot->store(b, std::memory_order_relaxed);
    }
    return b;
}

// Persistent grid: enough 256-thread workgroups to give each of `waves`
// wave tiles its own wave, capped at the number that can be resident on the
// device at once (CUs x resident workgroups per CU for this kernel).
template <class Kern>
int64_t persistent_grid(Kern kern, std::atomic<int> (&cache)[kMaxDevices], int64_t waves) {
    const int blocks_per_cu = cached_blocks_per_cu(kern, kThreads, cache);
    int64_t grid = (waves + kWavesPerGroup - 1) / kWavesPerGroup;
    const int64_t cap = static_cast<int64_t>(device_cu_count()) * blocks_per_cu;
    if (grid > cap) grid = cap;
    return grid < 1 ? 1 : grid;
}

}  // namespace kbit
