// Read-bandwidth probe (a measurement aid, not a step of the method).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace kldk {

// Reads n_rows rows of row_bytes (a multiple of 16) from a and, if b is not
// null, from b, with waves_per_row (1 or 4) waves per row; sink[r] = XOR of
// the 32-bit words of row r of both. start / stop (may be null): events the
// first and the last launch record themselves (hipExtLaunchKernel).
hipError_t launch_read_probe(const void* a, const void* b, int64_t n_rows, int64_t row_bytes, int waves_per_row,
                             uint32_t* sink, hipStream_t stream, hipEvent_t start = nullptr,
                             hipEvent_t stop = nullptr);

}  // namespace kldk
