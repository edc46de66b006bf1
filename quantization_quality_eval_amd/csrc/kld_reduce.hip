// Deterministic two-level reduction of the per-token results to the summaries
// the pages report: mean KLD and the same-top-1 fraction over every evaluated
// token ("Raw benchmark data" table of the Qwen3.6 27B quantization benchmark;
// "Quality" section of the GSQ-RCO model card), the max KLD and its row, and
// the sums behind the token-conditioned metrics of the same table and section
// (log-probability of the next token under each model, its probability
// change and that change squared, over the scored rows).
//
// The rows to reduce form one or more segments (a whole evaluation, or one
// summary per context, chunk or domain, which the model card reports per
// domain over fixed-length chunks). Every segment is cut into tiles of 1024
// rows counted from its first row.
// Level 1: one block per tile; each of its 256 threads folds 4 consecutive
// rows in order, then a fixed LDS tree combines the threads (float64 sums,
// (max, lowest row), int64 counts). Level 2: one block per segment folds that
// segment's tile partials the same way. A segment's result depends only on its
// rows' per-token values, never on how the rows were chunked or on which
// streams produced them; the whole-evaluation summary is the one-segment case.
// Work is O(n) bytes of per-token data (18 B per row), negligible next to the
// rows themselves.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kld_eval.h"
#include "kld_kernels.h"

namespace kldk {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerThread = 4;
static_assert(kThreads * kRowsPerThread == kReduceTileRows, "tile size");

__device__ __forceinline__ Partial identity() {
    Partial p;
    p.kld_sum = 0.0;
    p.kld_max = -INFINITY;
    p.kld_max_row = INT64_MAX;
    p.n_match = 0;
    p.logp_b_sum = 0.0;
    p.logp_q_sum = 0.0;
    p.dp_sum = 0.0;
    p.dp2_sum = 0.0;
    p.n_scored = 0;
    p.n_invalid = 0;
    return p;
}

__device__ __forceinline__ void take_max(Partial& a, double v, int64_t row) {
    if (v > a.kld_max || (v == a.kld_max && row < a.kld_max_row)) {
        a.kld_max = v;
        a.kld_max_row = row;
    }
}

__device__ __forceinline__ void combine(Partial& a, const Partial& b) {
    a.kld_sum += b.kld_sum;
    a.n_match += b.n_match;
    take_max(a, b.kld_max, b.kld_max_row);
    a.logp_b_sum += b.logp_b_sum;
    a.logp_q_sum += b.logp_q_sum;
    a.dp_sum += b.dp_sum;
    a.dp2_sum += b.dp2_sum;
    a.n_scored += b.n_scored;
    a.n_invalid += b.n_invalid;
}

__device__ __forceinline__ void fold_row(Partial& p, const RowIn& in, int64_t r) {
    const double v = static_cast<double>(in.kld[r]);
    p.kld_sum += v;
    p.n_match += in.match[r];
    take_max(p, v, r);
    if (!in.tok_state) return;  // no token arrays: nothing scored
    const uint8_t ts = in.tok_state[r];
    if (ts == 1) {
        const double d = static_cast<double>(in.dp[r]);
        p.logp_b_sum += static_cast<double>(in.logp_b[r]);
        p.logp_q_sum += static_cast<double>(in.logp_q[r]);
        p.dp_sum += d;
        p.dp2_sum += d * d;
        p.n_scored += 1;
    } else if (ts == 2) {
        p.n_invalid += 1;
    }
}

__device__ void block_tree(Partial& p, Partial* sm) {
    const int t = threadIdx.x;
    sm[t] = p;
    __syncthreads();
    for (int s = kThreads / 2; s > 0; s >>= 1) {
        if (t < s) {
            Partial a = sm[t];
            combine(a, sm[t + s]);
            sm[t] = a;
        }
        __syncthreads();
    }
    p = sm[0];
}

// tiles null: one segment [0, n_rows), block b folds tile tile0 + b, rows
// [(tile0 + b) kReduceTileRows, min(n_rows, (tile0 + b + 1) kReduceTileRows)),
// the same rows the host's tile list gives that segment.
__global__ void __launch_bounds__(kThreads)
    reduce_level1(RowIn in, const ReduceTile* __restrict__ tiles, int64_t tile0, int64_t n_rows, Partial* parts) {
    __shared__ Partial sm[kThreads];
    ReduceTile tile;
    if (tiles) {
        tile = tiles[blockIdx.x];
    } else {
        tile.start = (tile0 + blockIdx.x) * kReduceTileRows;
        tile.end = tile.start + kReduceTileRows < n_rows ? tile.start + kReduceTileRows : n_rows;
    }
    Partial p = identity();
    const int64_t r0 = tile.start + static_cast<int64_t>(threadIdx.x) * kRowsPerThread;
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i) {
        const int64_t r = r0 + i;
        if (r < tile.end) fold_row(p, in, r);
    }
    block_tree(p, sm);
    if (threadIdx.x == 0) parts[blockIdx.x] = p;
}

// seg_tile null: one segment whose partials are parts[0, n_tiles), of n_rows
// rows; its public summary goes to pub (when not null), the sums to result
// (when not null).
__global__ void __launch_bounds__(kThreads)
    reduce_level2(const Partial* __restrict__ parts, const int64_t* __restrict__ seg_tile,
                  const int64_t* __restrict__ seg_rows, DevSummary* result, int64_t n_tiles, int64_t n_rows,
                  kld_eval_summary* pub) {
    __shared__ Partial sm[kThreads];
    const int64_t s = blockIdx.x;
    const int64_t t0 = seg_tile ? seg_tile[s] : 0, t1 = seg_tile ? seg_tile[s + 1] : n_tiles;
    Partial p = identity();
    for (int64_t i = t0 + threadIdx.x; i < t1; i += kThreads) combine(p, parts[i]);
    block_tree(p, sm);
    if (threadIdx.x == 0) {
        const int64_t rows = seg_rows ? seg_rows[s] : n_rows;
        if (pub) {  // as the host forms it from the same sums (rows >= 1 here)
            const double n = static_cast<double>(rows);
            kld_eval_summary o;
            o.n_rows = rows;
            o.kld_sum = p.kld_sum;
            o.kld_mean = p.kld_sum / n;
            o.kld_max = p.kld_max;
            o.kld_max_row = p.kld_max_row;
            o.n_match = p.n_match;
            o.same_top1 = static_cast<double>(p.n_match) / n;
            pub[s] = o;
        }
        if (!result) return;
        DevSummary d;
        d.kld_sum = p.kld_sum;
        d.kld_max = p.kld_max;
        d.kld_max_row = p.kld_max_row;
        d.n_match = p.n_match;
        d.n_rows = rows;
        d.logp_b_sum = p.logp_b_sum;
        d.logp_q_sum = p.logp_q_sum;
        d.dp_sum = p.dp_sum;
        d.dp2_sum = p.dp2_sum;
        d.n_scored = p.n_scored;
        d.n_invalid = p.n_invalid;
        result[s] = d;
    }
}

// One segment [0, n_rows) in a single launch: every block folds its tile as
// reduce_level1 does; the last block to finish then folds all the partials as
// reduce_level2 does. Each block publishes its partial with an agent-scope
// release fence before taking a ticket from `done`; the block that draws the
// last ticket acquires before reading the partials and resets `done`.
__global__ void __launch_bounds__(kThreads)
    reduce_fused(RowIn in, int64_t n_rows, int64_t n_tiles, Partial* parts, unsigned int* done, DevSummary* result,
                 kld_eval_summary* pub) {
    __shared__ Partial sm[kThreads];
    __shared__ int sm_last;
    const int64_t start = static_cast<int64_t>(blockIdx.x) * kReduceTileRows;
    const int64_t end = start + kReduceTileRows < n_rows ? start + kReduceTileRows : n_rows;
    Partial p = identity();
    const int64_t r0 = start + static_cast<int64_t>(threadIdx.x) * kRowsPerThread;
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i) {
        const int64_t r = r0 + i;
        if (r < end) fold_row(p, in, r);
    }
    block_tree(p, sm);
    if (threadIdx.x == 0) {
        parts[blockIdx.x] = p;
        __threadfence();
        const unsigned int prev = atomicAdd(done, 1u);
        sm_last = prev == static_cast<unsigned int>(n_tiles - 1);
    }
    __syncthreads();
    if (!sm_last) return;
    __threadfence();
    Partial q = identity();
    for (int64_t i = threadIdx.x; i < n_tiles; i += kThreads) combine(q, parts[i]);
    block_tree(q, sm);
    if (threadIdx.x == 0) {
        *done = 0u;
        const double n = static_cast<double>(n_rows);
        if (pub) {  // as reduce_level2 forms it
            kld_eval_summary o;
            o.n_rows = n_rows;
            o.kld_sum = q.kld_sum;
            o.kld_mean = q.kld_sum / n;
            o.kld_max = q.kld_max;
            o.kld_max_row = q.kld_max_row;
            o.n_match = q.n_match;
            o.same_top1 = static_cast<double>(q.n_match) / n;
            *pub = o;
        }
        if (result) {
            DevSummary d;
            d.kld_sum = q.kld_sum;
            d.kld_max = q.kld_max;
            d.kld_max_row = q.kld_max_row;
            d.n_match = q.n_match;
            d.n_rows = n_rows;
            d.logp_b_sum = q.logp_b_sum;
            d.logp_q_sum = q.logp_q_sum;
            d.dp_sum = q.dp_sum;
            d.dp2_sum = q.dp2_sum;
            d.n_scored = q.n_scored;
            d.n_invalid = q.n_invalid;
            *result = d;
        }
    }
}

}  // namespace

int64_t reduce_fused_max_tiles() { return max_blocks_per_launch(kThreads); }

hipError_t launch_reduce_fused(const RowIn& in, int64_t n_rows, Partial* partials, unsigned int* done,
                               DevSummary* result, void* summary, hipStream_t stream) {
    const int64_t n_tiles = (n_rows + kReduceTileRows - 1) / kReduceTileRows;
    if (n_tiles < 1 || n_tiles > reduce_fused_max_tiles()) return hipErrorInvalidValue;
    hipLaunchKernelGGL(reduce_fused, dim3(static_cast<unsigned>(n_tiles)), dim3(kThreads), 0, stream, in, n_rows,
                       n_tiles, partials, done, result, static_cast<kld_eval_summary*>(summary));
    return hipGetLastError();
}

hipError_t launch_reduce(const RowIn& in, const ReduceTile* tiles, int64_t n_tiles, const int64_t* seg_tile,
                         const int64_t* seg_rows, int64_t n_segments, Partial* partials, DevSummary* result,
                         hipStream_t stream) {
    const int64_t per = max_blocks_per_launch(kThreads);
    for (int64_t done = 0; done < n_tiles; done += per) {
        const int64_t n = n_tiles - done < per ? n_tiles - done : per;
        hipLaunchKernelGGL(reduce_level1, dim3(static_cast<unsigned>(n)), dim3(kThreads), 0, stream, in, tiles + done,
                           int64_t{0}, int64_t{0}, partials + done);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // seg_tile holds absolute tile numbers, so a piece of the segment list
    // reads the same partials
    for (int64_t done = 0; done < n_segments; done += per) {
        const int64_t n = n_segments - done < per ? n_segments - done : per;
        hipLaunchKernelGGL(reduce_level2, dim3(static_cast<unsigned>(n)), dim3(kThreads), 0, stream, partials,
                           seg_tile + done, seg_rows + done, result + done, int64_t{0}, int64_t{0},
                           static_cast<kld_eval_summary*>(nullptr));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_reduce_whole(const RowIn& in, int64_t n_rows, Partial* partials, void* summary,
                               hipStream_t stream) {
    const int64_t n_tiles = (n_rows + kReduceTileRows - 1) / kReduceTileRows;
    const int64_t per = max_blocks_per_launch(kThreads);
    for (int64_t done = 0; done < n_tiles; done += per) {
        const int64_t n = n_tiles - done < per ? n_tiles - done : per;
        hipLaunchKernelGGL(reduce_level1, dim3(static_cast<unsigned>(n)), dim3(kThreads), 0, stream, in,
                           static_cast<const ReduceTile*>(nullptr), done, n_rows, partials + done);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(reduce_level2, dim3(1), dim3(kThreads), 0, stream, static_cast<const Partial*>(partials),
                       static_cast<const int64_t*>(nullptr), static_cast<const int64_t*>(nullptr),
                       static_cast<DevSummary*>(nullptr), n_tiles, n_rows, static_cast<kld_eval_summary*>(summary));
    return hipGetLastError();
}

}  // namespace kldk
