// Host-side launch geometry shared by the HIP translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"
#include "kbit_internal.h"

namespace kbit {

// Persistent grid: enough 256-thread workgroups to give each of `waves`
// wave tiles its own wave, capped at the number that can be resident on the
// device at once (CUs x resident workgroups per CU for this kernel).  The
// per-kernel residency is computed once and cached in `blocks_per_cu`.
template <class Kern>
int64_t persistent_grid(Kern kern, int& blocks_per_cu, int64_t waves) {
    if (blocks_per_cu == 0) {
        int b = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, kern, kThreads, 0) != hipSuccess || b < 1) b = 1;
        blocks_per_cu = b;
    }
    int64_t grid = (waves + kWavesPerGroup - 1) / kWavesPerGroup;
    const int64_t cap = static_cast<int64_t>(device_cu_count()) * blocks_per_cu;
    if (grid > cap) grid = cap;
    return grid < 1 ? 1 : grid;
}

}  // namespace kbit
