// Read-bandwidth probe: the attainable HBM read rate for the row kernels'
// access pattern, measured on the same buffers.
//
// One workgroup of NW waves (1 or 4) per row (or row pair): wave w reads the
// 1 KiB tiles w, w + NW, w + 2 NW, ... of each row with 16-byte non-temporal
// loads per lane, four tiles per row in flight, the shapes in which the row
// kernel streams its inputs (one wave per row for bf16 pairs in large
// handles, four otherwise), but with no arithmetic beyond an XOR of the
// words read. The XOR of a row's words is written out, so that the loads
// cannot be removed and the result can be checked on the host.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kld_kernels.h"
#include "kld_probe.h"

namespace kldk {
namespace {

constexpr int kProbeU = 4;  // tiles per row in flight per wave

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

template <bool kTwo, int kProbeWaves>
__global__ void __launch_bounds__(kProbeWaves * 64)
    kld_read_probe_kernel(const u32x4* __restrict__ a, const u32x4* __restrict__ b, int64_t row_vecs,
                          uint32_t* __restrict__ sink) {
    __shared__ uint32_t wx[kProbeWaves];
    const int64_t r = blockIdx.x;
    const u32x4* ra = a + r * row_vecs;
    const u32x4* rb = kTwo ? b + r * row_vecs : nullptr;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t tiles = row_vecs / 64;
    uint32_t acc = 0;
    int64_t k = wave;
    for (; k + static_cast<int64_t>(kProbeU - 1) * kProbeWaves < tiles; k += kProbeU * kProbeWaves) {
        u32x4 va[kProbeU], vb[kProbeU];
#pragma unroll
        for (int u = 0; u < kProbeU; ++u) {
            va[u] = __builtin_nontemporal_load(ra + (k + u * kProbeWaves) * 64 + lane);
            if (kTwo) vb[u] = __builtin_nontemporal_load(rb + (k + u * kProbeWaves) * 64 + lane);
        }
#pragma unroll
        for (int u = 0; u < kProbeU; ++u) acc ^= fold(va[u]) ^ (kTwo ? fold(vb[u]) : 0u);
    }
    for (; k < tiles; k += kProbeWaves) {
        acc ^= fold(__builtin_nontemporal_load(ra + k * 64 + lane));
        if (kTwo) acc ^= fold(__builtin_nontemporal_load(rb + k * 64 + lane));
    }
    const int64_t tail = tiles * 64 + threadIdx.x;  // fewer than 64 vectors remain
    if (tail < row_vecs) {
        acc ^= fold(ra[tail]);
        if (kTwo) acc ^= fold(rb[tail]);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o);
    if (lane == 0) wx[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t x = 0;
#pragma unroll
        for (int w = 0; w < kProbeWaves; ++w) x ^= wx[w];
        sink[r] = x;
    }
}

template <int NW>
hipError_t launch_shape(const void* a, const void* b, int64_t n_rows, int64_t row_bytes, uint32_t* sink,
                        hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    const int64_t row_vecs = row_bytes / 16;
    const int64_t per = max_blocks_per_launch(NW * 64);
    for (int64_t done = 0; done < n_rows; done += per) {
        const int64_t n = n_rows - done < per ? n_rows - done : per;
        const u32x4* pa = static_cast<const u32x4*>(a) + done * row_vecs;
        const u32x4* pb = b ? static_cast<const u32x4*>(b) + done * row_vecs : nullptr;
        hipEvent_t e0 = done == 0 ? start : nullptr, e1 = done + n == n_rows ? stop : nullptr;
        if (b)
            hipExtLaunchKernelGGL((kld_read_probe_kernel<true, NW>), dim3(static_cast<unsigned>(n)), dim3(NW * 64),
                                  0, stream, e0, e1, 0, pa, pb, row_vecs, sink + done);
        else
            hipExtLaunchKernelGGL((kld_read_probe_kernel<false, NW>), dim3(static_cast<unsigned>(n)), dim3(NW * 64),
                                  0, stream, e0, e1, 0, pa, pb, row_vecs, sink + done);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_read_probe(const void* a, const void* b, int64_t n_rows, int64_t row_bytes, int waves_per_row,
                             uint32_t* sink, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    if (waves_per_row == 1) return launch_shape<1>(a, b, n_rows, row_bytes, sink, stream, start, stop);
    if (waves_per_row == 4) return launch_shape<4>(a, b, n_rows, row_bytes, sink, stream, start, stop);
    return hipErrorInvalidValue;
}

}  // namespace kldk
