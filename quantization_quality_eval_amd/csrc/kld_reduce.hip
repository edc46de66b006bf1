// Deterministic two-level reduction of the per-token results to the summary
// the pages report: mean KLD and the same-top-1 fraction over every evaluated
// token ("Raw benchmark data" table of the Qwen3.6 27B quantization benchmark;
// "Quality" section of the GSQ-RCO model card), plus the max KLD and its row.
//
// Level 1: block b owns the fixed row range [b * 1024, (b + 1) * 1024). Each
// of its 256 threads folds 4 consecutive rows in order, then a fixed LDS tree
// combines the threads: float64 sum, (max, lowest row) and an int64 match
// count. Level 2: one block folds the level-1 partials in index order the
// same way. The result depends only on the per-token arrays, never on how the
// rows were chunked or on which streams produced them. Work is O(n) bytes of
// per-token data (5 B per row), negligible next to the rows themselves.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kld_kernels.h"

namespace kldk {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerThread = 4;
constexpr int kRowsPerBlock = kThreads * kRowsPerThread;  // 1024

struct Part {
    double sum;
    double mx;
    int64_t mx_row;
    int64_t match;
};

__device__ __forceinline__ void take_max(Part& a, double v, int64_t row) {
    if (v > a.mx || (v == a.mx && row < a.mx_row)) {
        a.mx = v;
        a.mx_row = row;
    }
}

__device__ __forceinline__ void combine(Part& a, const Part& b) {
    a.sum += b.sum;
    a.match += b.match;
    take_max(a, b.mx, b.mx_row);
}

__device__ void block_tree(Part& p, Part* sm) {
    const int t = threadIdx.x;
    sm[t] = p;
    __syncthreads();
    for (int s = kThreads / 2; s > 0; s >>= 1) {
        if (t < s) {
            Part a = sm[t];
            combine(a, sm[t + s]);
            sm[t] = a;
        }
        __syncthreads();
    }
    p = sm[0];
}

__global__ void __launch_bounds__(kThreads)
    reduce_level1(const float* __restrict__ kld, const uint8_t* __restrict__ match, int64_t n_rows,
                  double* part_sum, double* part_max, int64_t* part_max_row, int64_t* part_match) {
    __shared__ Part sm[kThreads];
    const int64_t b = blockIdx.x;
    Part p{0.0, -INFINITY, INT64_MAX, 0};
    const int64_t r0 = b * kRowsPerBlock + static_cast<int64_t>(threadIdx.x) * kRowsPerThread;
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i) {
        const int64_t r = r0 + i;
        if (r < n_rows) {
            const double v = static_cast<double>(kld[r]);
            p.sum += v;
            p.match += match[r];
            take_max(p, v, r);
        }
    }
    block_tree(p, sm);
    if (threadIdx.x == 0) {
        part_sum[b] = p.sum;
        part_max[b] = p.mx;
        part_max_row[b] = p.mx_row;
        part_match[b] = p.match;
    }
}

__global__ void __launch_bounds__(kThreads)
    reduce_level2(const double* __restrict__ part_sum, const double* __restrict__ part_max,
                  const int64_t* __restrict__ part_max_row, const int64_t* __restrict__ part_match,
                  int64_t n_parts, int64_t n_rows, DevSummary* result) {
    __shared__ Part sm[kThreads];
    Part p{0.0, -INFINITY, INT64_MAX, 0};
    for (int64_t i = threadIdx.x; i < n_parts; i += kThreads) {
        Part q{part_sum[i], part_max[i], part_max_row[i], part_match[i]};
        combine(p, q);
    }
    block_tree(p, sm);
    if (threadIdx.x == 0) {
        result->kld_sum = p.sum;
        result->kld_max = p.mx;
        result->kld_max_row = p.mx_row;
        result->n_match = p.match;
        result->n_rows = n_rows;
    }
}

}  // namespace

int64_t reduce_partials(int64_t n_rows) { return (n_rows + kRowsPerBlock - 1) / kRowsPerBlock; }

hipError_t launch_reduce(const float* kld, const uint8_t* match, int64_t n_rows, double* part_sum,
                         double* part_max, int64_t* part_max_row, int64_t* part_match, DevSummary* result,
                         hipStream_t stream) {
    const int64_t n_parts = reduce_partials(n_rows);
    hipLaunchKernelGGL(reduce_level1, dim3(static_cast<unsigned>(n_parts)), dim3(kThreads), 0, stream, kld, match,
                       n_rows, part_sum, part_max, part_max_row, part_match);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(reduce_level2, dim3(1), dim3(kThreads), 0, stream, part_sum, part_max, part_max_row,
                       part_match, n_parts, n_rows, result);
    return hipGetLastError();
}

}  // namespace kldk
