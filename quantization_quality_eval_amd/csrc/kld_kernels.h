// Internal interface between the C-ABI host code and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kldk {

enum ElemType : int { kF32 = 0, kBF16 = 1 };

// Per-token destinations. The handle arrays are indexed by row_offset + r,
// the optional caller arrays by r.
struct RowOut {
    float* kld;
    uint8_t* match;
    int32_t* argmax_b;
    int32_t* argmax_q;
    float* lse_b;
    float* lse_q;
    float* kld_out;
    uint8_t* match_out;
    int32_t* argmax_b_out;
    int32_t* argmax_q_out;
};

// Device-side summary written by the second reduction level.
struct DevSummary {
    double kld_sum;
    double kld_max;
    int64_t kld_max_row;
    int64_t n_match;
    int64_t n_rows;
};

// Launch the fused per-row kernel over n_rows row pairs (one workgroup each).
// shape_rows (the handle's row capacity) selects the launch shape.
hipError_t launch_rows(int base_type, int quant_type, const void* base, const void* quant,
                       int64_t vocab, int64_t n_rows, int64_t row_offset, int64_t shape_rows,
                       const RowOut& out, hipStream_t stream);

// Number of first-level partials needed to reduce n_rows per-token values.
int64_t reduce_partials(int64_t n_rows);

// Two-level deterministic reduction of handle rows [0, n_rows).
hipError_t launch_reduce(const float* kld, const uint8_t* match, int64_t n_rows,
                         double* part_sum, double* part_max, int64_t* part_max_row,
                         int64_t* part_match, DevSummary* result, hipStream_t stream);

}  // namespace kldk
