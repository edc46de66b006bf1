// Read-bandwidth probe (a measurement aid, not a step of the method).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace kldk {

// Reads n_rows rows of row_bytes (a multiple of 16) from a and, if b is not
// null, from b; sink[r] = XOR of the 32-bit words of row r of both.
hipError_t launch_read_probe(const void* a, const void* b, int64_t n_rows, int64_t row_bytes, uint32_t* sink,
                             hipStream_t stream);

}  // namespace kldk
