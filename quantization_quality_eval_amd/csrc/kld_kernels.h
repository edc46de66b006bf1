// Internal interface between the C-ABI host code and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kldk {

enum ElemType : int { kF32 = 0, kBF16 = 1 };

// The dispatch packet holds a launch's grid size in work-items as a 32-bit
// value: launchers keep workgroups x threads per workgroup within INT32_MAX
// and cut larger grids into pieces of at most this many workgroups.
constexpr int64_t max_blocks_per_launch(int threads_per_block) { return int64_t{INT32_MAX} / threads_per_block; }

// Per-token destinations. The handle arrays are indexed by row_offset + r,
// the optional caller arrays by r. `tokens` (optional, indexed by r) holds the
// id of the token that follows each position; without it every row gets
// token state 0 (not scored). The row kernel needs kld and match; it skips
// argmax_b / argmax_q / lse_b / lse_q when null, and the four token arrays
// (tok_state, logp_b, logp_q, dp: all set or all null) when tok_state is null.
struct RowOut {
    float* kld;
    uint8_t* match;
    int32_t* argmax_b;
    int32_t* argmax_q;
    double* lse_b;  // float64 log-normalisers (kept for the gradient)
    double* lse_q;
    float* logp_b;
    float* logp_q;
    float* dp;
    uint8_t* tok_state;  // 0 not scored, 1 scored, 2 id >= vocab
    uint8_t* retake;     // row pass: conditioning flags (kRowFlag*), nonzero where the row was taken again
    double* topk_coef;   // top-K rows: P + R, (P + R) Q_rest - R and lse_rest per row, NaN if bad (may be null)
    const int32_t* tokens;
    float* kld_out;
    uint8_t* match_out;
    int32_t* argmax_b_out;
    int32_t* argmax_q_out;
    float* logp_b_out;
    float* logp_q_out;
    float* dp_out;
};

// Per-token arrays the reduction reads (handle buffers). With tok_state null
// the token arrays are not read and every row counts as not scored.
struct RowIn {
    const float* kld;
    const uint8_t* match;
    const float* logp_b;
    const float* logp_q;
    const float* dp;
    const uint8_t* tok_state;
};

// Sums over a set of rows, written by the second reduction level.
struct DevSummary {
    double kld_sum;
    double kld_max;
    int64_t kld_max_row;  // INT64_MAX when the set is empty
    int64_t n_match;
    int64_t n_rows;
    double logp_b_sum;
    double logp_q_sum;
    double dp_sum;
    double dp2_sum;
    int64_t n_scored;
    int64_t n_invalid;
};

// One level-1 tile: rows [start, end) of one segment.
struct ReduceTile {
    int64_t start;
    int64_t end;
};

// Level-1 partial, one per tile (layout private to kld_reduce.hip).
struct Partial {
    double kld_sum;
    double kld_max;
    int64_t kld_max_row;
    int64_t n_match;
    double logp_b_sum;
    double logp_q_sum;
    double dp_sum;
    double dp2_sum;
    int64_t n_scored;
    int64_t n_invalid;
};

// Conditioning flags the row pass writes per row (RowOut::retake). A row with
// any bit set was evaluated a second time in float64 by its own workgroup:
// the fp32 sums' rounding is amplified past the divergence's tolerance, the
// quant normaliser has lost bits to cancellation, or a rescale moved more
// mass between the sums than the normaliser's bound allows.
constexpr unsigned int kRowFlagAmplified = 1u;
constexpr unsigned int kRowFlagQuantMass = 2u;
constexpr unsigned int kRowFlagCarried = 4u;

// Launch the fused per-row kernel over n_rows row pairs (one workgroup each).
// shape_rows (the handle's row capacity) selects the launch shape.
// n_rows must not exceed rows_max_per_launch(); callers cut larger calls.
// start / stop (may be null): events the dispatch itself records when the
// kernel begins and ends (hipExtLaunchKernel), with no packets of their own.
hipError_t launch_rows(int base_type, int quant_type, const void* base, const void* quant,
                       int64_t vocab, int64_t n_rows, int64_t row_offset, int64_t shape_rows,
                       const RowOut& out, hipStream_t stream, hipEvent_t start = nullptr,
                       hipEvent_t stop = nullptr);
int64_t rows_max_per_launch();

// Gradient of the per-token KL with respect to the quantized logits,
// scale * (q - p), for n_rows rows whose float64 log-normalisers are
// lse_b/lse_q[row_offset + r]; grad is [n_rows, vocab] of grad_type.
hipError_t launch_grad(int base_type, int quant_type, int grad_type, const void* base, const void* quant,
                       const double* lse_b, const double* lse_q, int64_t vocab, int64_t n_rows, int64_t row_offset,
                       float scale, void* grad, hipStream_t stream);

// Top-K + rest-of-mass form of base rows (k in [1, topk_max_k()], k <= vocab):
// idx_out/logp_out [n_rows, k], rest_out [n_rows].
int topk_max_k();
hipError_t launch_topk_compress(int base_type, const void* base, int64_t vocab, int64_t n_rows, int k,
                                int32_t* idx_out, float* logp_out, float* rest_out, hipStream_t stream);

// LDS bytes the evaluation kernel needs besides its vocab-bit map.
constexpr int64_t kTopkEvalStaticLds = 4096;
// Coarsened KL of full quant rows from stored top-K rows, written like the row
// kernel's results (handle rows row_offset + r, optional caller copies).
hipError_t launch_topk_eval(int quant_type, const int32_t* idx, const float* logp, const float* rest, int k,
                            const void* quant, int64_t vocab, int64_t n_rows, int64_t row_offset, const RowOut& out,
                            hipStream_t stream);

// Gradient of the coarsened top-K KL with respect to the quantized logits for
// rows already evaluated by launch_topk_eval (their lse_q and the two
// coefficients saved at row_offset + r); grad is [n_rows, vocab] of grad_type.
hipError_t launch_topk_grad(int quant_type, int grad_type, const int32_t* idx, const float* logp, int k,
                            const void* quant, int64_t vocab, int64_t n_rows, int64_t row_offset,
                            const double* lse_q, const double* coef, float scale, void* grad, hipStream_t stream);

// dst[i] = (float)src[i], i < n.
hipError_t launch_lse_to_f32(const double* src, float* dst, int64_t n, hipStream_t stream);

// Rows per level-1 tile; segments are cut into tiles of this many rows from
// their first row.
constexpr int64_t kReduceTileRows = 1024;

// Two-level deterministic reduction. Level 1 folds each tile of `tiles`
// (device, n_tiles entries) into partials[tile]; level 2 folds, for segment s,
// the partials [seg_tile[s], seg_tile[s + 1]) (device, n_segments + 1
// entries) into result[s]. `seg_rows` (device, n_segments) gives each
// segment's row count.
hipError_t launch_reduce(const RowIn& in, const ReduceTile* tiles, int64_t n_tiles, const int64_t* seg_tile,
                         const int64_t* seg_rows, int64_t n_segments, Partial* partials, DevSummary* result,
                         hipStream_t stream);

// The same two levels over one segment of rows [0, n_rows) with no tables:
// level 1 cuts it into tiles of kReduceTileRows rows from row 0 (the tiles
// launch_reduce is given for that segment), level 2 folds every partial and
// writes the public summary struct (kld_eval_summary of kld_eval.h) to
// `summary`, whose fields equal what the host derives from the same sums.
// partials holds ceil(n_rows / kReduceTileRows) entries.
hipError_t launch_reduce_whole(const RowIn& in, int64_t n_rows, Partial* partials, void* summary,
                               hipStream_t stream);

// The same single segment in one launch: the level-1 blocks of
// launch_reduce_whole, of which the last to finish (a device counter `done`,
// zero before the launch and zero again after it) folds every partial in the
// level-2 order and writes the sums to `result` and/or the public summary to
// `summary` (either may be null, either may be host-mapped memory).
// Bit-identical to launch_reduce over the same segment. Needs
// ceil(n_rows / kReduceTileRows) <= reduce_fused_max_tiles().
int64_t reduce_fused_max_tiles();
hipError_t launch_reduce_fused(const RowIn& in, int64_t n_rows, Partial* partials, unsigned int* done,
                               DevSummary* result, void* summary, hipStream_t stream);

}  // namespace kldk
