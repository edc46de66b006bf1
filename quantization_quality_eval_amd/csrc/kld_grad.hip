// Gradient of the per-token KL(P_base || Q_quant) with respect to the
// quantized logits, and the float32 export of the log-normalisers.
//
// The GSQ-RCO model card ("How it was made" step 7) tunes the quantized model
// by minimising KL(BF16 || quantized) of the next-token distributions; the
// backward pass of that loss starts from dKL/dz_quant[i] = q_i - p_i (the
// derivative of log-sum-exp is the softmax), times the row's weight in the
// loss. This kernel is that backward step: it re-reads both rows and uses the
// float64 log-normalisers the row kernel saved in the handle, so it needs no
// reduction of its own and is a pure stream: read two rows, write one.
//
// Decomposition: one workgroup of 256 threads per (row, chunk of 2048 or 4096
// elements); each thread takes groups of 8 elements (non-temporal loads of
// both rows), computes both probabilities and writes the gradient with
// non-temporal stores; the lane layout depends on the output type (see
// Layout). Rows whose shape or alignment rules out vector access take an
// element-wise path.
//
// Numerics (fp32 per element): with S the float nearest the float64
// log-normaliser L and c = (L - S) log2(e) (|c| <= 2^-24 |L| log2 e),
//   p = 2^fma(zb - S_b, log2 e, -c_b),  q likewise,  g = w (q - p).
// z - S is exact for bf16 inputs near the top of the row (and off by at most
// half an ulp of the difference otherwise), so p carries a relative error of
// about |z - L| 2^-24 plus the normaliser's own, which is what the parity
// tolerance states.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "kld_bf16_pairs.h"
#include "kld_kernels.h"

namespace kldk {
namespace {

constexpr float kLog2eF = 1.44269504088896340736f;
constexpr double kLog2eD = 1.44269504088896340736;
constexpr int kThreads = 256;
#ifndef KLD_GRAD_NT
#define KLD_GRAD_NT 1  // non-temporal stores
#endif

// Lane layout and work per thread, by output type (measured on MI355X,
// 8192 x 151936 bf16 rows): a float32 gradient is written best when a lane's
// 8 elements are two runs of 4, 256 apart, so that every store instruction of
// a wave writes one contiguous 1 KiB (two 16-byte stores per lane 16 bytes
// apart leave each instruction half of every line and cost 11% extra write
// traffic); one group of 8 per thread. A bfloat16 gradient (one 16-byte store
// per lane) is written best with 8 consecutive elements per lane, two groups
// per thread.
template <class EG>
struct Layout {
    static constexpr bool kSplit = true;
    static constexpr int kGroups = 1;
};
template <>
struct Layout<uint16_t> {
    static constexpr bool kSplit = false;
    static constexpr int kGroups = 2;
};
template <class EG>
constexpr int chunk_elems() {
    return kThreads * 8 * Layout<EG>::kGroups;  // elements per workgroup
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float widen(float x) { return x; }
__device__ __forceinline__ float widen(uint16_t b) { return __uint_as_float(static_cast<unsigned int>(b) << 16); }

// 8 consecutive elements, 16-byte aligned.
__device__ __forceinline__ void load8(const uint16_t* p, float (&z)[8]) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        z[2 * k] = __uint_as_float(v[k] << 16);
        z[2 * k + 1] = __uint_as_float(v[k] & 0xffff0000u);
    }
}
__device__ __forceinline__ void load8(const float* p, float (&z)[8]) {
    const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + 1);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        z[k] = a[k];
        z[4 + k] = b[k];
    }
}

// float -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ unsigned int to_bf16(float x) {
    const unsigned int u = __float_as_uint(x);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <class T>
__device__ __forceinline__ void st(T v, T* p) {
#if KLD_GRAD_NT
    __builtin_nontemporal_store(v, p);
#else
    *p = v;
#endif
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Two runs of 4 elements: [p, p + 4) and [p + 256, p + 260); each run is
// checked against the end of the chunk on its own.
__device__ __forceinline__ void load44(const uint16_t* p, bool ok0, bool ok1, float (&z)[8]) {
    u32x2 a = {0u, 0u}, b = {0u, 0u};
    if (ok0) a = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    if (ok1) b = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p + 256));
    z[0] = __uint_as_float(a[0] << 16); z[1] = __uint_as_float(a[0] & 0xffff0000u);
    z[2] = __uint_as_float(a[1] << 16); z[3] = __uint_as_float(a[1] & 0xffff0000u);
    z[4] = __uint_as_float(b[0] << 16); z[5] = __uint_as_float(b[0] & 0xffff0000u);
    z[6] = __uint_as_float(b[1] << 16); z[7] = __uint_as_float(b[1] & 0xffff0000u);
}
__device__ __forceinline__ void load44(const float* p, bool ok0, bool ok1, float (&z)[8]) {
    f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
    if (ok0) a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    if (ok1) b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 256));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        z[k] = a[k];
        z[4 + k] = b[k];
    }
}
__device__ __forceinline__ void store44(float* p, bool ok0, bool ok1, const float (&g)[8]) {
    const f32x4 a = {g[0], g[1], g[2], g[3]}, b = {g[4], g[5], g[6], g[7]};
    if (ok0) st(a, reinterpret_cast<f32x4*>(p));
    if (ok1) st(b, reinterpret_cast<f32x4*>(p + 256));
}

__device__ __forceinline__ void store8(uint16_t* p, const float (&g)[8]) {
    u32x4 v;
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = to_bf16(g[2 * k]) | (to_bf16(g[2 * k + 1]) << 16);
    st(v, reinterpret_cast<u32x4*>(p));
}

__device__ __forceinline__ void store1(float* p, float g) { *p = g; }
__device__ __forceinline__ void store1(uint16_t* p, float g) { *p = static_cast<uint16_t>(to_bf16(g)); }

struct Shift {
    float s;  // float nearest the log-normaliser
    float c;  // (L - s) log2(e)
};

__device__ __forceinline__ Shift make_shift(double L) {
    const float s = static_cast<float>(L);
    return Shift{s, static_cast<float>((L - static_cast<double>(s)) * kLog2eD)};
}

__device__ __forceinline__ float prob(float z, const Shift& sh) {
    return __builtin_amdgcn_exp2f(fmaf(z - sh.s, kLog2eF, -sh.c));
}

template <class EB, class EQ, class EG>
__global__ void __launch_bounds__(kThreads)
    kld_grad_kernel(const EB* __restrict__ base, const EQ* __restrict__ quant, const double* __restrict__ lse_b,
                    const double* __restrict__ lse_q, int64_t vocab, int64_t row_offset, int chunks_per_row,
                    int vec_ok, float scale, EG* __restrict__ grad) {
    const int64_t bid = blockIdx.x;
    const int64_t r = bid / chunks_per_row;
    const int64_t c = bid - r * chunks_per_row;
    const Shift sb = make_shift(lse_b[row_offset + r]);
    const Shift sq = make_shift(lse_q[row_offset + r]);
    const EB* rb = base + r * vocab;
    const EQ* rq = quant + r * vocab;
    EG* rg = grad + r * vocab;
    constexpr int kChunk = chunk_elems<EG>();
    constexpr int kGroupsPerThread = Layout<EG>::kGroups;
    const int64_t c0 = c * kChunk;
    const int64_t c1 = min(vocab, c0 + kChunk);
    if constexpr (std::is_same<EB, uint16_t>::value && std::is_same<EQ, uint16_t>::value) {
        if (vec_ok) {
            // both rows bf16: the loads stay packed and z - s comes from
            // v_dot2_f32_bf16 on the pairs (pairs::shifted_tile), one
            // instruction per element instead of an unpack and a subtraction
            unsigned int slo, shi;
            asm volatile("v_mov_b32 %0, %1" : "=v"(slo) : "s"(0x00003f80u));  // bf16 pair (1, 0)
            asm volatile("v_mov_b32 %0, %1" : "=v"(shi) : "s"(0x3f800000u));  // bf16 pair (0, 1)
            auto probs = [&](const pairs::u32x4& raw, const Shift& sh, float (&pr)[8]) {
                float x[8];
                pairs::shifted_tile(raw, slo, shi, -sh.s, x);
#pragma unroll
                for (int k = 0; k < 8; ++k) pr[k] = __builtin_amdgcn_exp2f(fmaf(x[k], kLog2eF, -sh.c));
            };
            pairs::u32x4 xb[kGroupsPerThread], xq[kGroupsPerThread];
            if constexpr (Layout<EG>::kSplit) {
                const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
                for (int u = 0; u < kGroupsPerThread; ++u) {
                    const int64_t i = c0 + static_cast<int64_t>(u * 4 + wave) * 512 + 4 * lane;
                    u32x2 b0 = {0u, 0u}, b1 = {0u, 0u}, q0 = {0u, 0u}, q1 = {0u, 0u};
                    if (i < c1) {
                        b0 = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(rb + i));
                        q0 = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(rq + i));
                    }
                    if (i + 256 < c1) {
                        b1 = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(rb + i + 256));
                        q1 = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(rq + i + 256));
                    }
                    xb[u] = pairs::u32x4{b0[0], b0[1], b1[0], b1[1]};
                    xq[u] = pairs::u32x4{q0[0], q0[1], q1[0], q1[1]};
                }
#pragma unroll
                for (int u = 0; u < kGroupsPerThread; ++u) {
                    const int64_t i = c0 + static_cast<int64_t>(u * 4 + wave) * 512 + 4 * lane;
                    float pb[8], pq[8], g[8];
                    probs(xb[u], sb, pb);
                    probs(xq[u], sq, pq);
#pragma unroll
                    for (int k = 0; k < 8; ++k) g[k] = scale * (pq[k] - pb[k]);
                    store44(rg + i, i < c1, i + 256 < c1, g);
                }
            } else {
#pragma unroll
                for (int u = 0; u < kGroupsPerThread; ++u) {
                    const int64_t i = c0 + (static_cast<int64_t>(u) * kThreads + threadIdx.x) * 8;
                    if (i < c1) {
                        xb[u] = __builtin_nontemporal_load(reinterpret_cast<const pairs::u32x4*>(rb + i));
                        xq[u] = __builtin_nontemporal_load(reinterpret_cast<const pairs::u32x4*>(rq + i));
                    }
                }
#pragma unroll
                for (int u = 0; u < kGroupsPerThread; ++u) {
                    const int64_t i = c0 + (static_cast<int64_t>(u) * kThreads + threadIdx.x) * 8;
                    if (i < c1) {
                        float pb[8], pq[8], g[8];
                        probs(xb[u], sb, pb);
                        probs(xq[u], sq, pq);
#pragma unroll
                        for (int k = 0; k < 8; ++k) g[k] = scale * (pq[k] - pb[k]);
                        store8(rg + i, g);
                    }
                }
            }
            return;
        }
    }
    if (vec_ok) {
        float zb[kGroupsPerThread][8], zq[kGroupsPerThread][8];
        if constexpr (Layout<EG>::kSplit) {
            // group u of wave w covers [c0 + (u * 4 + w) * 512, + 512): lane l
            // owns elements 4l .. 4l + 3 and 256 + 4l .. 256 + 4l + 3 of it, so
            // every load and store instruction of the wave is one contiguous span
            const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
            for (int u = 0; u < kGroupsPerThread; ++u) {
                const int64_t i = c0 + static_cast<int64_t>(u * 4 + wave) * 512 + 4 * lane;
                load44(rb + i, i < c1, i + 256 < c1, zb[u]);
                load44(rq + i, i < c1, i + 256 < c1, zq[u]);
            }
#pragma unroll
            for (int u = 0; u < kGroupsPerThread; ++u) {
                const int64_t i = c0 + static_cast<int64_t>(u * 4 + wave) * 512 + 4 * lane;
                float g[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) g[k] = scale * (prob(zq[u][k], sq) - prob(zb[u][k], sb));
                store44(rg + i, i < c1, i + 256 < c1, g);
            }
        } else {
#pragma unroll
            for (int u = 0; u < kGroupsPerThread; ++u) {
                const int64_t i = c0 + (static_cast<int64_t>(u) * kThreads + threadIdx.x) * 8;
                if (i < c1) {
                    load8(rb + i, zb[u]);
                    load8(rq + i, zq[u]);
                }
            }
#pragma unroll
            for (int u = 0; u < kGroupsPerThread; ++u) {
                const int64_t i = c0 + (static_cast<int64_t>(u) * kThreads + threadIdx.x) * 8;
                if (i < c1) {
                    float g[8];
#pragma unroll
                    for (int k = 0; k < 8; ++k) g[k] = scale * (prob(zq[u][k], sq) - prob(zb[u][k], sb));
                    store8(rg + i, g);
                }
            }
        }
    } else {
        for (int64_t i = c0 + threadIdx.x; i < c1; i += kThreads)
            store1(rg + i, scale * (prob(widen(rq[i]), sq) - prob(widen(rb[i]), sb)));
    }
}

template <class EB, class EQ, class EG>
hipError_t launch_grad_typed(const void* base, const void* quant, const double* lse_b, const double* lse_q,
                             int64_t vocab, int64_t n_rows, int64_t row_offset, float scale, void* grad,
                             hipStream_t stream) {
    constexpr int kChunk = chunk_elems<EG>();
    const int64_t cpr = (vocab + kChunk - 1) / kChunk;
    const bool vec_ok = vocab % 8 == 0 && reinterpret_cast<uintptr_t>(base) % 16 == 0 &&
                        reinterpret_cast<uintptr_t>(quant) % 16 == 0 && reinterpret_cast<uintptr_t>(grad) % 16 == 0;
    const int64_t rows_per_launch = max_blocks_per_launch(kThreads) / cpr;
    for (int64_t done = 0; done < n_rows; done += rows_per_launch) {
        const int64_t n = min(rows_per_launch, n_rows - done);
        hipLaunchKernelGGL((kld_grad_kernel<EB, EQ, EG>), dim3(static_cast<unsigned>(n * cpr)), dim3(kThreads), 0,
                           stream, static_cast<const EB*>(base) + done * vocab,
                           static_cast<const EQ*>(quant) + done * vocab, lse_b, lse_q, vocab, row_offset + done,
                           static_cast<int>(cpr), vec_ok ? 1 : 0, scale, static_cast<EG*>(grad) + done * vocab);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <class EB, class EQ>
hipError_t launch_grad_out(int grad_type, const void* base, const void* quant, const double* lse_b,
                           const double* lse_q, int64_t vocab, int64_t n_rows, int64_t row_offset, float scale,
                           void* grad, hipStream_t stream) {
    if (grad_type == kF32)
        return launch_grad_typed<EB, EQ, float>(base, quant, lse_b, lse_q, vocab, n_rows, row_offset, scale, grad,
                                                stream);
    return launch_grad_typed<EB, EQ, uint16_t>(base, quant, lse_b, lse_q, vocab, n_rows, row_offset, scale, grad,
                                               stream);
}

__global__ void __launch_bounds__(kThreads) lse_to_f32_kernel(const double* __restrict__ src, float* __restrict__ dst,
                                                              int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (i < n) dst[i] = static_cast<float>(src[i]);
}

}  // namespace

hipError_t launch_grad(int base_type, int quant_type, int grad_type, const void* base, const void* quant,
                       const double* lse_b, const double* lse_q, int64_t vocab, int64_t n_rows, int64_t row_offset,
                       float scale, void* grad, hipStream_t stream) {
    if (base_type == kBF16 && quant_type == kBF16)
        return launch_grad_out<uint16_t, uint16_t>(grad_type, base, quant, lse_b, lse_q, vocab, n_rows, row_offset,
                                                   scale, grad, stream);
    if (base_type == kF32 && quant_type == kF32)
        return launch_grad_out<float, float>(grad_type, base, quant, lse_b, lse_q, vocab, n_rows, row_offset, scale,
                                             grad, stream);
    if (base_type == kF32 && quant_type == kBF16)
        return launch_grad_out<float, uint16_t>(grad_type, base, quant, lse_b, lse_q, vocab, n_rows, row_offset,
                                                scale, grad, stream);
    return launch_grad_out<uint16_t, float>(grad_type, base, quant, lse_b, lse_q, vocab, n_rows, row_offset, scale,
                                            grad, stream);
}

hipError_t launch_lse_to_f32(const double* src, float* dst, int64_t n, hipStream_t stream) {
    for (int64_t done = 0; done < n; done += int64_t{1} << 30) {
        const int64_t m = min(int64_t{1} << 30, n - done);
        hipLaunchKernelGGL(lse_to_f32_kernel, dim3(static_cast<unsigned>((m + kThreads - 1) / kThreads)),
                           dim3(kThreads), 0, stream, src + done, dst + done, m);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace kldk
