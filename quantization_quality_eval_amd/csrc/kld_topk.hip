// Base rows stored as their top-K tokens plus the rest of the mass, and the
// divergence of a full quantized row from such a row.
//
// The GSQ-RCO model card ("How it was made" step 7) tunes against the BF16
// model's "top-128 distributions (and the rest of the mass)": per position the
// K most probable tokens with their probabilities and the total probability of
// all other tokens. Stored form per row here: K indices (the K largest logits,
// equal logits by lowest index, most probable first -- so the first is the
// argmax), their log-probabilities z - lse (float32), and the rest mass
// (float32), summed over the other tokens directly. The divergence of a full
// quantized row from a stored row is the KL of both distributions coarsened
// to the same K + 1 outcomes (the K stored tokens and "any other token"):
//   KL_K = sum_k p_k (log p_k - log q_k) + R (log R - log Q_rest),
// which is the full KL when K = V and never exceeds it.
//
// topk_compress_kernel (one workgroup of 256 threads per base row): a pass
// over a sample of the row (every 4th step for K <= 256, every 2nd for larger
// K) keeps each thread's largest values, whose K-th largest bounds the row's
// K-th largest logit from below; a full pass collects the elements at or
// above it (the candidates) and sums the exponentials of all others; a radix
// select of the K-th largest candidate and a sort of those at or above it
// pick the stored tokens -- 1.25 (1.5) reads of the row.
// Rows with more candidates than the LDS lists hold take the exact path:
//   1. radix select of the K-th largest order-preserving key, 8 bits per pass
//      (2 passes for bf16 keys, 4 for f32), histograms in LDS; the first pass
//      also finds the row maximum M;
//   2. one gather pass in index order: a block-wide scan of per-thread counts
//      places every element above the threshold, and the first ties at it, at
//      a position that depends only on its index (deterministic), while the
//      exponentials are summed separately for stored tokens, exp(z - M), and
//      for the rest, exp(z - threshold) (fp32 sums of 8, accumulated in
//      float64; a rest sum too small to be accurate is taken again);
//   3. a sort in LDS of the elements above the threshold (value descending,
//      index ascending); the ties follow in index order.
// topk_grad_kernel: the gradient of KL_K with respect to the quantized
// logits, one chunk of a row per workgroup (see the kernel).
// topk_eval_kernel (one workgroup of 256 threads per quantized row):
//   1. the stored indices become a bitmap in LDS (V bits);
//   2. one streaming pass over the quantized row: per thread the running
//      maximum (rescaling in float64 when it grows), the lowest index of the
//      maximum, and the mass of the tokens outside the bitmap;
//   3. the stored tokens' logits are gathered and their terms evaluated in
//      float64. Only the streamed rest mass carries fp32 rounding -- relative
//      error about 1.33e-7 per nat of its terms' mass-weighted mean distance
//      below the row maximum, plus 5.4e-7; a mass under (V - K) e^-60, where
//      terms could flush, is summed again relative to its own maximum -- and
//      it enters KL_K with the coefficient Q_rest - R, which vanishes as the
//      quantized row approaches the base row.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "kld_bf16_pairs.h"
#include "kld_kernels.h"

namespace kldk {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
#ifndef KLD_TOPK_EVAL_U
#define KLD_TOPK_EVAL_U 1  // 8-element groups per thread per step, evaluation stream
#endif
#ifndef KLD_TOPK_COMPRESS_U
#define KLD_TOPK_COMPRESS_U 1  // 8-element groups per thread per step, compression passes
#endif
constexpr float kLog2eF = 1.44269504088896340736f;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float widen(float x) { return x; }
__device__ __forceinline__ float widen(uint16_t b) { return __uint_as_float(static_cast<unsigned int>(b) << 16); }

// Raw 8-element groups: loaded first, widened at use, so that several loads
// can be in flight before the first one is needed. load() is non-temporal
// (data read once); load_temporal() leaves the lines cached for a second
// read shortly after.
template <class E>
struct Raw8;
template <>
struct Raw8<uint16_t> {
    u32x4 v;
    __device__ __forceinline__ void load(const uint16_t* p) {
        v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    }
    __device__ __forceinline__ void load_temporal(const uint16_t* p) { v = *reinterpret_cast<const u32x4*>(p); }
    __device__ __forceinline__ void unpack(float (&z)[8]) const {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            z[2 * k] = __uint_as_float(v[k] << 16);
            z[2 * k + 1] = __uint_as_float(v[k] & 0xffff0000u);
        }
    }
};
template <>
struct Raw8<float> {
    f32x4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
        b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + 1);
    }
    __device__ __forceinline__ void load_temporal(const float* p) {
        a = *reinterpret_cast<const f32x4*>(p);
        b = *(reinterpret_cast<const f32x4*>(p) + 1);
    }
    __device__ __forceinline__ void unpack(float (&z)[8]) const {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            z[k] = a[k];
            z[4 + k] = b[k];
        }
    }
};

// Visit every 8-element group of a row (vocab % 8 == 0, 16-byte aligned) in
// steps of kThreads x 8 x kU elements: thread t takes groups t, t + kThreads,
// ... of each step, in ascending order. Full steps go through a ring of two
// register sets -- while one step is processed the loads of the next are in
// flight; the steady loop is unrolled twice so that both sets have
// compile-time names and every load in it is unconditional. f(i0, z, valid)
// is called for every group slot of every step (valid false past the row's
// end in the last, partial step), so a caller may synchronize inside f.
// With kStride > 1 only the full steps 0, kStride, 2 kStride, ... are visited
// (a sample of the row; the partial step only when there is no full step).
// kRaw: f receives the group's Raw8 (not yet widened) instead of z.
// kTemporal: the full steps are loaded with load_temporal().
template <int kU, int kStride = 1, bool kRaw = false, bool kTemporal = false, class E, class F>
__device__ __forceinline__ void stream_groups(const E* row, int64_t vocab, int t, F&& f) {
    constexpr int64_t kStep = static_cast<int64_t>(kThreads) * 8 * kU;
    const int64_t n_full = vocab / kStep;
    const int64_t ns = (n_full + kStride - 1) / kStride;  // visited full steps
    Raw8<E> ra[kU], rb[kU];
    auto load_step = [&](Raw8<E>(&rr)[kU], int64_t si) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const E* p = row + si * kStride * kStep + (static_cast<int64_t>(u) * kThreads + t) * 8;
            if constexpr (kTemporal)
                rr[u].load_temporal(p);
            else
                rr[u].load(p);
        }
    };
    auto take_step = [&](const Raw8<E>(&rr)[kU], int64_t si) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t i0 = si * kStride * kStep + (static_cast<int64_t>(u) * kThreads + t) * 8;
            if constexpr (kRaw) {
                f(i0, rr[u], true);
            } else {
                float z[8];
                rr[u].unpack(z);
                f(i0, z, true);
            }
        }
    };
    if (ns >= 2) {
        load_step(ra, 0);
        load_step(rb, 1);
        int64_t si = 0;
        for (; si + 3 < ns; si += 2) {
            take_step(ra, si);
            load_step(ra, si + 2);
            take_step(rb, si + 1);
            load_step(rb, si + 3);
        }
        // steps si and si + 1 are loaded; at most one more remains
        take_step(ra, si);
        if (si + 2 < ns) load_step(ra, si + 2);
        take_step(rb, si + 1);
        if (si + 2 < ns) take_step(ra, si + 2);
    } else if (ns == 1) {
        load_step(ra, 0);
        take_step(ra, 0);
    }
    const int64_t full = n_full * kStep;
    if (full < vocab && (kStride == 1 || n_full == 0)) {  // last, partial step: every slot is visited, loads are guarded
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t i0 = full + (static_cast<int64_t>(u) * kThreads + t) * 8;
            const bool ok = i0 < vocab;
            Raw8<E> r{};
            if (ok) r.load(row + i0);
            if constexpr (kRaw) {
                f(i0, r, ok);
            } else {
                float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                if (ok) r.unpack(z);
                f(i0, z, ok);
            }
        }
    }
}

// Order-preserving unsigned key of a finite float; -0 and +0 share a key.
__device__ __forceinline__ uint32_t order_key(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) == 0u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// Block sums of N values per thread, in a fixed order: a butterfly inside
// each wave, then the waves in order through sm[N * kWaves]; one barrier
// (plus one before sm is reused). Every thread returns the same totals.
template <int N>
__device__ __forceinline__ void block_sum(double (&v)[N], double* sm) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] += __shfl_xor(v[i], o);
    }
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) {
#pragma unroll
        for (int i = 0; i < N; ++i) sm[N * w + i] = v[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < N; ++i) {
        v[i] = 0.0;
#pragma unroll
        for (int j = 0; j < kWaves; ++j) v[i] += sm[N * j + i];
    }
}

// Block-wide exclusive scan of a packed pair of counts (low and high 16 bits)
// in thread order; `tot` receives the block total. wsum is double-buffered by
// the caller's chunk parity, so one barrier per call suffices.
__device__ __forceinline__ uint32_t block_scan2(uint32_t c, uint32_t* wsum, uint32_t& tot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    uint32_t before = 0;
    tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const uint32_t s = wsum[w];
        if (w < wave) before += s;
        tot += s;
    }
    return before + incl - c;
}

// ----------------------------------------------------- far rest masses ---
// A streamed sum W = sum_i exp(-d_i) of N fp32 exponentials, d_i >= 0 the
// distance below the shift, has relative error about 1.33e-7 d_i per term
// (the fp32 argument (z - shift) log2(e) is rounded relative to its size)
// plus ~5.4e-7 (the exponential's ulp and sums of 8), and terms with
// d_i > 87.3 flush to zero. The mass-weighted mean of the d_i is at most
// ln(N / W) (largest when all terms are equal), so W >= N e^-C bounds the
// relative error by 1.33e-7 C + 5.4e-7 and makes the flushed part
// negligible for C well below 87. Sums under that bound are taken again by
// sum_exp_below, relative to the terms' own maximum.
constexpr double kFarCompress = 2.0611536224385579e-09;  // e^-20: the stored rest mass within 3.2e-6
constexpr double kFarEval = 8.7565107626965203e-27;      // e^-60: the quantized rest mass, no flushing

// sum of exp(z_i - S) over the row's elements i with below(z_i, i), taken
// relative to their maximum Mr -- one pass for Mr, one for the fp32 sum of
// exp(z_i - Mr) (the largest term is exactly 1, so the mean distance is at
// most ln N) -- times exp(Mr - S) in float64; 0 when no element qualifies.
// Every thread of the block calls it (it synchronizes) and gets the same value.
template <class E, class Below>
__device__ __forceinline__ double sum_exp_below(const E* row, int64_t vocab, int vec_ok, double S, Below below,
                                             float* wmax, double* sm) {
    const int t = threadIdx.x;
    auto visit = [&](auto&& g) {  // one group at a time: a rare path, kept light on registers
        if (vec_ok) {
            for (int64_t i0 = 8 * static_cast<int64_t>(t); i0 < vocab; i0 += 8 * kThreads) {
                Raw8<E> raw;
                raw.load(row + i0);
                float z[8];
                raw.unpack(z);
                g(i0, z, 8);
            }
        } else {
            for (int64_t i0 = t; i0 < vocab; i0 += kThreads) {
                const float z = widen(row[i0]);
                g(i0, &z, 1);
            }
        }
    };
    float mr = -INFINITY;
    visit([&](int64_t i0, const float* z, int nz) {
        for (int j = 0; j < nz; ++j)
            if (below(z[j], i0 + j)) mr = fmaxf(mr, z[j]);
    });
    mr = wave_max(mr);
    __syncthreads();  // wmax may still be read from an earlier use
    if ((t & 63) == 0) wmax[t >> 6] = mr;
    __syncthreads();
    float Mr = wmax[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) Mr = fmaxf(Mr, wmax[w]);
    if (Mr == -INFINITY) return 0.0;  // the same in every thread
    double acc[1] = {0.0};
    visit([&](int64_t i0, const float* z, int nz) {
        float s = 0.0f;
        for (int j = 0; j < nz; ++j)
            if (below(z[j], i0 + j)) s += __builtin_amdgcn_exp2f((z[j] - Mr) * kLog2eF);
        acc[0] += static_cast<double>(s);
    });
    block_sum<1>(acc, sm);
    return acc[0] * exp(static_cast<double>(Mr) - S);
}

// ------------------------------------------------------------ compress ---

constexpr int kMaxK = 1024;
constexpr int kCandCap = 2048;  // candidates the sampled-bound selection can hold per row
constexpr int kWaveCap = kCandCap / kWaves;  // ... in one list per wave
static_assert(kWaveCap % kThreads == 0, "a thread's slots t + j kThreads must not straddle two lists");
#ifndef KLD_TOPK_SAMPLE_STRIDE
#define KLD_TOPK_SAMPLE_STRIDE 4  // the bound's sample: every 4th step of the row
#endif
#ifndef KLD_TOPK_SAMPLE_TOP
#define KLD_TOPK_SAMPLE_TOP 2  // largest values kept per thread in the sample
#endif
constexpr int kSampleStride = KLD_TOPK_SAMPLE_STRIDE;
constexpr int kSampleTop = KLD_TOPK_SAMPLE_TOP;

// Bitonic sort of a[0, n) in LDS, descending, by the whole thread block;
// a[n, next power of two) must hold values that sort last. Ends synchronized.
template <class T>
__device__ void block_sort_desc(T* a, uint32_t n) {
    uint32_t P = 1;
    while (P < n) P <<= 1;
    for (uint32_t size = 2; size <= P; size <<= 1) {
        for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
            for (uint32_t i = threadIdx.x; i < P / 2; i += kThreads) {
                const uint32_t lo = 2 * i - (i & (stride - 1));
                const uint32_t hi = lo + stride;
                const bool desc = (lo & size) == 0;
                const T x = a[lo], y = a[hi];
                if ((x < y) == desc) {
                    a[lo] = y;
                    a[hi] = x;
                }
            }
            __syncthreads();
        }
    }
}

// Sort of n <= 2 kThreads distinct keys a[0, n) in LDS, descending, by rank:
// a key's place is the number of keys larger than it. Thread t ranks entries
// t and t + kThreads; every thread reads all n keys in the same order, so each
// read is a single broadcast address per wave. a must be visible to every
// thread on entry. Ends synchronized.
__device__ __forceinline__ void block_rank_sort_desc(uint64_t* a, uint32_t n) {
    const uint32_t t = threadIdx.x;
    const uint64_t e0 = t < n ? a[t] : 0ull;
    uint32_t r0 = 0;
    if (n <= static_cast<uint32_t>(kThreads)) {
#pragma unroll 8
        for (uint32_t j = 0; j < n; ++j) r0 += a[j] > e0 ? 1u : 0u;
        __syncthreads();
        if (t < n) a[r0] = e0;
    } else {
        const uint64_t e1 = t + kThreads < n ? a[t + kThreads] : 0ull;
        uint32_t r1 = 0;
#pragma unroll 8
        for (uint32_t j = 0; j < n; ++j) {
            const uint64_t x = a[j];
            r0 += x > e0 ? 1u : 0u;
            r1 += x > e1 ? 1u : 0u;
        }
        __syncthreads();
        a[r0] = e0;  // t < kThreads < n
        if (t + kThreads < n) a[r1] = e1;
    }
    __syncthreads();
}

// Sort of n distinct keys a[0, n) in LDS, descending: by rank up to
// 2 kThreads keys, otherwise bitonic over the next power of two (a must have
// room for it; the padding is written here). a must be visible to every
// thread on entry. Ends synchronized.
__device__ __forceinline__ void sort_keys_desc(uint64_t* a, uint32_t n) {
    if (n <= 2u * kThreads) {
        block_rank_sort_desc(a, n);
        return;
    }
    uint32_t P = 1;
    while (P < n) P <<= 1;
    for (uint32_t i = n + threadIdx.x; i < P; i += kThreads) a[i] = 0ull;  // padding sorts last
    __syncthreads();
    block_sort_desc(a, n);
}

// Radix select by the whole block: the key T of the k-th largest of the
// significant keys (8 x kDigits bits) that the threads hold -- each thread's
// keys are those that keys(f) passes to f -- for 1 <= k <= their number;
// 8-bit digits from the top, histograms in hist[256]; n_greater receives how
// many keys exceed T. Wave 0 finds each digit with a scan over its lanes'
// bins. sel[2] is scratch. Ends synchronized.
template <int kDigits, class Keys>
__device__ __forceinline__ uint32_t block_select(Keys keys, uint32_t k, uint32_t* hist, uint32_t* sel,
                                                 uint32_t& n_greater) {
    const int t = threadIdx.x;
    uint32_t prefix = 0, pmask = 0, need = k;
    for (int d = 0; d < kDigits; ++d) {
        const int shift = (kDigits - 1 - d) * 8;
        hist[t] = 0u;
        __syncthreads();
        keys([&](uint32_t s) {
            if ((s & pmask) == prefix) atomicAdd(&hist[(s >> shift) & 255u], 1u);
        });
        __syncthreads();
        if (t < 64) {
            // lane l holds bins 255 - 4 l .. 252 - 4 l: counts from the top
            uint32_t c[4], sum = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                c[j] = hist[255 - 4 * t - j];
                sum += c[j];
            }
            uint32_t incl = sum;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t y = __shfl_up(incl, o);
                if (t >= o) incl += y;
            }
            uint32_t cum = incl - sum;
            if (cum < need && need <= incl) {  // the digit lies in this lane's bins
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (cum < need && need <= cum + c[j]) {
                        sel[0] = static_cast<uint32_t>(255 - 4 * t - j);
                        sel[1] = need - cum;
                    }
                    cum += c[j];
                }
            }
        }
        __syncthreads();
        prefix |= sel[0] << shift;
        pmask |= 255u << shift;
        need = sel[1];
    }
    n_greater = k - need;
    return prefix;
}

// Waves per SIMD: five for the small-K form (its 21 KB of LDS allows it and
// its registers fit in 96), four for the large-K form (its 38 KB of LDS
// holds it there).
template <class EB, bool kLarge>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kLarge ? 4 : 5)))
    topk_compress_kernel(const EB* __restrict__ base, int64_t vocab, int k, int vec_ok, int32_t* __restrict__ idx_out,
                         float* __restrict__ logp_out, float* __restrict__ rest_out) {
    constexpr bool kBf16 = std::is_same<EB, uint16_t>::value;
    constexpr int kDigits = kBf16 ? 2 : 4;   // 8-bit digits of the significant key bits
    constexpr int kLowBits = kBf16 ? 16 : 0;  // key bits a bfloat16 never sets
    // sampled-bound selection: k <= kThreads (kLarge false) or k <= kMaxK
    // (kLarge: a denser sample, more values kept per thread, longer lists)
    constexpr int kCap = kLarge ? 2 * kCandCap : kCandCap;  // candidates held per row
    constexpr int kWCap = kCap / kWaves;                     // ... in one list per wave
    constexpr int kStride = kLarge ? 2 : kSampleStride;
    constexpr int kTop = kLarge ? 8 : kSampleTop;
    constexpr int kSampledMaxK = kLarge ? kMaxK : kThreads;
    static_assert(kWCap % kThreads == 0, "a thread's slots t + j kThreads must not straddle two lists");
    static_assert(kSampledMaxK <= kThreads * kTop, "the bound needs k kept values");
    __shared__ uint32_t hist[256];
    __shared__ uint32_t sh_sel[3];            // digit, prefix, still needed
    __shared__ uint64_t above[kCap];      // (key << 32) | ~index: candidates (kWaves lists of kWCap; while the
                                          // full pass appends them, the value's raw bits in place of its key),
                                          // or elements above the threshold
    __shared__ int32_t ties[kMaxK];           // indices at the threshold, in index order
    __shared__ uint32_t wsum[2][kWaves];
    __shared__ float wmax[kWaves];
    __shared__ double dsum[3 * kWaves];
    __shared__ uint32_t wcand[kWaves];        // candidates found by each wave

    const int t = threadIdx.x;
    const int64_t r = blockIdx.x;
    const EB* row = base + r * vocab;

    // ---- sampled bound + one full pass (k <= kSampledMaxK) ----
    // Any k distinct elements of the row bound its k-th largest logit from
    // below. A first, sampled pass reads every kStride-th step and keeps
    // each thread's kTop largest values; the k-th largest of those is a
    // bound T0, so every stored token (ties included) is among the elements
    // >= T0 (T0 by a radix select over the kept values). One full pass then
    // collects those candidates (about k x kStride) and sums exp(z - T0)
    // over all the others, which are rest mass for certain and lie below T0
    // (shifting by T0 rather than by a maximum keeps the largest of these
    // terms' fp32 arguments small; a sum too small for the bound above
    // kFarCompress is taken again). A second radix select finds the k-th
    // largest candidate value; the candidates at or above it are moved to
    // the front and sorted by (value, index), the first k are stored, every
    // other candidate joins the rest mass, in float64 relative to the row
    // maximum max(Ms, best candidate), Ms the sample's. A wave with more
    // candidates than its list holds (long runs of equal logits) sends the
    // row to the exact radix select below.
    if (k <= kSampledMaxK) {
        float top[kTop];
#pragma unroll
        for (int c = 0; c < kTop; ++c) top[c] = -INFINITY;
        auto keep = [&](float x) {  // insert into the descending top list
            if (kTop > 2 && !(x > top[kTop - 1])) return;  // long lists: most values fall short at once
#pragma unroll
            for (int c = 0; c < kTop; ++c) {
                const float hi = fmaxf(top[c], x);
                x = fminf(top[c], x);
                top[c] = hi;
            }
        };
        if (vec_ok) {
            // temporal loads: the full pass reads these steps again shortly
            // after and finds them in cache (its own loads stay non-temporal)
            stream_groups<KLD_TOPK_COMPRESS_U, kStride, false, true>(
                row, vocab, t, [&](int64_t, const float* z, bool ok) {
                    if (ok)
#pragma unroll
                        for (int j = 0; j < 8; ++j) keep(z[j]);
                });
        } else {
            for (int64_t i0 = t; i0 < vocab; i0 += kThreads) keep(widen(row[i0]));
        }
        const float wm_ = wave_max(top[0]);
        if ((t & 63) == 0) wmax[t >> 6] = wm_;
        __syncthreads();
        float M = wmax[0];  // the sample's maximum
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, wmax[w]);
        // T0: the k-th largest of the threads' kept values
        uint32_t n_gt0;
        const uint32_t T0k = block_select<kDigits>(
            [&](auto&& f) {
#pragma unroll
                for (int c = 0; c < kTop; ++c) f(order_key(top[c]) >> kLowBits);
            },
            static_cast<uint32_t>(k), hist, sh_sel, n_gt0);
        const float T0 = key_value(kLowBits ? ((T0k << kLowBits) | ((T0k & 0x8000u) ? 0u : 0xffffu)) : T0k);
        // Each wave appends its candidates to its own list of kWCap
        // entries: a ballot gives the wave's candidates of one slot, a lane's
        // place is its rank among them (mbcnt), and the wave's count wc is the
        // same in every lane that took part in every step -- lane 0 always
        // does, being the first of its wave in every step. No atomics.
        uint64_t* const wlist = above + (t >> 6) * kWCap;
        uint32_t wc = 0;
        double wr = 0.0;
        // The rest's exponent arguments in one fma: z log2(e) - T0L with T0L
        // = T0 log2(e) rounded once, i.e. (z - T0) log2(e) + dT plus the
        // fma's own rounding (half an ulp of the argument, as the product of
        // the exact difference had), where dT = T0 log2(e) - T0L is the same
        // for every term; the sum is scaled by 2^-dT once it is complete.
        const float T0L = T0 * kLog2eF;
        auto collect = [&](int64_t i0, const float* z, int nz) {
            float sr = 0.0f;
            for (int j = 0; j < nz; ++j) {
                const bool c = z[j] >= T0;
                const uint64_t mask = __ballot(c);
                if (mask) {
                    if (c) {
                        const uint32_t pos = wc + __builtin_amdgcn_mbcnt_hi(
                                                      static_cast<uint32_t>(mask >> 32),
                                                      __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
                        // the raw bits: the order-preserving key is formed once per
                        // candidate when the selection loads the lists, not here in
                        // every wave slot that holds one
                        if (pos < static_cast<uint32_t>(kWCap))
                            wlist[pos] = (static_cast<uint64_t>(__float_as_uint(z[j])) << 32) |
                                         static_cast<uint32_t>(~static_cast<uint32_t>(i0 + j));
                    }
                    wc += static_cast<uint32_t>(__popcll(mask));
                }
                if (!c) sr += __builtin_amdgcn_exp2f(fmaf(z[j], kLog2eF, -T0L));
            }
            wr += static_cast<double>(sr);
        };
        if (vec_ok) {
            stream_groups<KLD_TOPK_COMPRESS_U>(row, vocab, t, [&](int64_t i0, const float* z, bool ok) {
                if (ok) collect(i0, z, 8);
            });
        } else {
            for (int64_t i0 = t; i0 < vocab; i0 += kThreads) {
                const float z = widen(row[i0]);
                collect(i0, &z, 1);
            }
        }
        if ((t & 63) == 0) wcand[t >> 6] = wc;
        __syncthreads();
        uint32_t cnt[kWaves];
        bool fits = true;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            cnt[w] = wcand[w];
            fits = fits && cnt[w] <= static_cast<uint32_t>(kWCap);
        }
        if (fits) {
            // Thread t takes slots t + j kThreads of `above` (list
            // j kThreads / kWCap, place t + j kThreads % kWCap); a slot
            // holds a candidate when its place is below its list's count.
            constexpr int kPer = kCap / kThreads;
            uint64_t mine[kPer];
            uint32_t heldm = 0;
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const bool h = static_cast<uint32_t>(t + (j * kThreads) % kWCap) < cnt[(j * kThreads) / kWCap];
                const uint64_t e = above[t + j * kThreads];  // raw bits of the value, ~index
                mine[j] = h ? (static_cast<uint64_t>(order_key(__uint_as_float(static_cast<uint32_t>(e >> 32)))) << 32) |
                                  (e & 0xffffffffull)
                            : 0ull;
                heldm |= static_cast<uint32_t>(h) << j;
            }
            // the k-th largest candidate value Tc; the candidates at or above
            // it (k plus any further ties at Tc) are moved to the front of the
            // list and sorted, the others are rest mass
            uint32_t n_gt;
            const uint32_t Tc = block_select<kDigits>(
                [&](auto&& f) {
#pragma unroll
                    for (int j = 0; j < kPer; ++j)
                        if ((heldm >> j) & 1u) f(static_cast<uint32_t>(mine[j] >> 32) >> kLowBits);
                },
                static_cast<uint32_t>(k), hist, sh_sel, n_gt);
            uint32_t keepm = 0, n_keep = 0;
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                if (((heldm >> j) & 1u) && (static_cast<uint32_t>(mine[j] >> 32) >> kLowBits) >= Tc) {
                    keepm |= 1u << j;
                    ++n_keep;
                }
            }
            uint32_t m;
            uint32_t pos = block_scan2(n_keep, wsum[0], m);  // synchronizes: every entry is read
#pragma unroll
            for (int j = 0; j < kPer; ++j)
                if ((keepm >> j) & 1u) above[pos++] = mine[j];
            __syncthreads();
            sort_keys_desc(above, m);
            // the row maximum: the best candidate, unless the sample's maximum is larger
            const double Md = fmax(static_cast<double>(M),
                                   static_cast<double>(key_value(static_cast<uint32_t>(above[0] >> 32))));
            double wm = 0.0, wx = 0.0;
#pragma unroll
            for (int j = 0; j < kPer; ++j)
                if (((heldm & ~keepm) >> j) & 1u)
                    wx += exp(static_cast<double>(key_value(static_cast<uint32_t>(mine[j] >> 32))) - Md);
            for (uint32_t j = t; j < m; j += kThreads) {
                const double e = exp(static_cast<double>(key_value(static_cast<uint32_t>(above[j] >> 32))) - Md);
                if (j < static_cast<uint32_t>(k))
                    wm += e;
                else
                    wx += e;
            }
            double ws[3] = {wm, wx, wr};  // stored (rel. Md), other candidates (rel. Md), the rest (rel. T0)
            block_sum<3>(ws, dsum);
            if (ws[2] > 0.0) {  // undo the shared offset of the rest's arguments (the product is exact in float64)
                const double dT = static_cast<double>(T0) * static_cast<double>(kLog2eF) - static_cast<double>(T0L);
                ws[2] *= exp2(-dT);
            }
            int64_t n_far = vocab;  // elements below T0
#pragma unroll
            for (int w = 0; w < kWaves; ++w) n_far -= cnt[w];
            if (n_far > 0 && ws[2] < static_cast<double>(n_far) * kFarCompress)
                ws[2] = sum_exp_below(row, vocab, vec_ok, static_cast<double>(T0),
                                      [&](float z, int64_t) { return !(z >= T0); }, wmax, dsum);
            const double w_rest = ws[1] + (ws[2] > 0.0 ? ws[2] * exp(static_cast<double>(T0) - Md) : 0.0);
            const double wall = ws[0] + w_rest;
            const double lse = Md + log(wall);
            for (int j = t; j < k; j += kThreads) {
                const uint64_t e = above[j];
                idx_out[r * k + j] = static_cast<int32_t>(~static_cast<uint32_t>(e & 0xffffffffu));
                logp_out[r * k + j] =
                    static_cast<float>(static_cast<double>(key_value(static_cast<uint32_t>(e >> 32))) - lse);
            }
            if (t == 0) rest_out[r] = static_cast<float>(w_rest / wall);
            return;
        }
        __syncthreads();
    }

    // ---- exact radix select (a row with too many candidates) ----
    // 1. radix select (first pass also takes the maximum)
    uint32_t prefix = 0, pmask = 0, need = static_cast<uint32_t>(k);
    float lmax = -INFINITY;
    for (int d = 0; d < kDigits; ++d) {
        const int shift = (kDigits - 1 - d) * 8;
        hist[t] = 0u;
        __syncthreads();
        auto count = [&](const float* z, int nz) {
            for (int j = 0; j < nz; ++j) {
                if (d == 0) lmax = fmaxf(lmax, z[j]);
                const uint32_t s = order_key(z[j]) >> kLowBits;
                if ((s & pmask) == prefix) atomicAdd(&hist[(s >> shift) & 255u], 1u);
            }
        };
        if (vec_ok) {
            stream_groups<KLD_TOPK_COMPRESS_U>(row, vocab, t, [&](int64_t, const float* z, bool ok) {
                if (ok) count(z, 8);
            });
        } else {
            for (int64_t i0 = t; i0 < vocab; i0 += kThreads) {
                const float z = widen(row[i0]);
                count(&z, 1);
            }
        }
        __syncthreads();
        if (t == 0) {
            uint32_t cum = 0, digit = 0;
            for (int b = 255; b >= 0; --b) {
                if (cum + hist[b] >= need) {
                    digit = static_cast<uint32_t>(b);
                    break;
                }
                cum += hist[b];
            }
            sh_sel[0] = digit;
            sh_sel[2] = need - cum;
        }
        __syncthreads();
        prefix |= sh_sel[0] << shift;
        pmask |= 255u << shift;
        need = sh_sel[2];
        __syncthreads();
    }
    const uint32_t T = prefix;                  // threshold on the significant key bits
    const uint32_t n_above = static_cast<uint32_t>(k) - need;

    // row maximum
    lmax = wave_max(lmax);
    if ((t & 63) == 0) wmax[t >> 6] = lmax;
    __syncthreads();
    float M = wmax[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, wmax[w]);
    // the threshold's value: the shift of the rest mass (its largest terms
    // lie just below it), unless it is -inf (then the rest is zero mass)
    const float tie_value = key_value(kLowBits ? ((T << kLowBits) | ((T & 0x8000u) ? 0u : 0xffffu)) : T);
    const float Ts = tie_value > -INFINITY ? tie_value : M;

    // ---- 2. gather in index order, sums of exp(z - M) (stored) and exp(z - Ts) (rest) ----
    uint32_t above_base = 0, tie_base = 0;
    double w_mem = 0.0, w_rest = 0.0;
    uint32_t parity = 0;
    // one group of nz elements from index i0 (nz = 0 for an empty slot); every
    // thread calls this the same number of times (it synchronizes)
    auto gather = [&](int64_t i0, const float* z, int nz) {
        uint32_t gt = 0, eq = 0, ngt = 0, neq = 0;
        for (int j = 0; j < nz; ++j) {
            const uint32_t s = order_key(z[j]) >> kLowBits;
            if (s > T) {
                gt |= 1u << j;
                ++ngt;
            } else if (s == T) {
                eq |= 1u << j;
                ++neq;
            }
        }
        uint32_t tot;
        const uint32_t ex = block_scan2(ngt | (neq << 16), wsum[parity], tot);
        parity ^= 1u;
        uint32_t pa = above_base + (ex & 0xffffu), pt = tie_base + (ex >> 16);
        float sm = 0.0f, sr = 0.0f;
        for (int j = 0; j < nz; ++j) {
            bool member = false;
            if (gt & (1u << j)) {
                above[pa++] = (static_cast<uint64_t>(order_key(z[j])) << 32) |
                              static_cast<uint32_t>(~static_cast<uint32_t>(i0 + j));
                member = true;
            } else if (eq & (1u << j)) {
                if (pt < need) {
                    ties[pt] = static_cast<int32_t>(i0 + j);
                    member = true;
                }
                ++pt;
            }
            const float e = __builtin_amdgcn_exp2f((z[j] - (member ? M : Ts)) * kLog2eF);
            if (member)
                sm += e;
            else
                sr += e;
        }
        w_mem += static_cast<double>(sm);
        w_rest += static_cast<double>(sr);
        above_base += tot & 0xffffu;
        tie_base += tot >> 16;
    };
    if (vec_ok) {
        stream_groups<KLD_TOPK_COMPRESS_U>(row, vocab, t,
                                           [&](int64_t i0, const float* z, bool ok) { gather(i0, z, ok ? 8 : 0); });
    } else {
        for (int64_t c0 = 0; c0 < vocab; c0 += kThreads) {
            const int64_t i0 = c0 + t;
            const float z = i0 < vocab ? widen(row[i0]) : 0.0f;
            gather(i0, &z, i0 < vocab ? 1 : 0);
        }
    }

    // ---- 3. order the elements above the threshold ----
    __syncthreads();
    sort_keys_desc(above, n_above);

    // ---- outputs ----
    double ws[2] = {w_mem, w_rest};
    block_sum<2>(ws, dsum);
    const int64_t n_rest = vocab - k;
    if (n_rest > 0 && ws[1] < static_cast<double>(n_rest) * kFarCompress) {
        // the ties past the k-th (1 each relative to the threshold) and the elements below it
        const double extra = Ts == tie_value ? static_cast<double>(tie_base - need) : 0.0;
        ws[1] = extra + sum_exp_below(row, vocab, vec_ok, static_cast<double>(Ts),
                                      [&](float z, int64_t) { return (order_key(z) >> kLowBits) < T; }, wmax, dsum);
    }
    const double wr = ws[1] > 0.0 ? ws[1] * exp(static_cast<double>(Ts) - static_cast<double>(M)) : 0.0;
    const double wall = ws[0] + wr;
    const double lse = static_cast<double>(M) + log(wall);
    for (int j = t; j < k; j += kThreads) {
        int32_t ix;
        float z;
        if (static_cast<uint32_t>(j) < n_above) {
            const uint64_t e = above[j];
            ix = static_cast<int32_t>(~static_cast<uint32_t>(e & 0xffffffffu));
            z = key_value(static_cast<uint32_t>(e >> 32));
        } else {
            ix = ties[j - n_above];
            z = tie_value;
        }
        idx_out[r * k + j] = ix;
        logp_out[r * k + j] = static_cast<float>(static_cast<double>(z) - lse);
    }
    if (t == 0) rest_out[r] = static_cast<float>(wr / wall);
}

// ---------------------------------------------------------------- eval ---

template <class EQ>
__global__ void __launch_bounds__(kThreads)
    topk_eval_kernel(const EQ* __restrict__ quant, const int32_t* __restrict__ sidx, const float* __restrict__ slogp,
                     const float* __restrict__ srest, int64_t vocab, int k, int vec_ok, int64_t row_offset,
                     RowOut out) {
    extern __shared__ uint32_t bitmap[];   // ceil(vocab / 32) words
    __shared__ double wred[kWaves][4];
    __shared__ double dres[kWaves];
    __shared__ float wmax[kWaves];
    __shared__ int widx[kWaves];

    const int t = threadIdx.x;
    const int64_t r = blockIdx.x;
    const EQ* row = quant + r * vocab;
    const int32_t* ix = sidx + r * k;
    const float* lp = slogp + r * k;
    const int64_t words = (vocab + 31) / 32;

    // ---- 1. bitmap of the stored tokens; out-of-range or repeated ids poison the row ----
    for (int64_t w = t; w < words; w += kThreads) bitmap[w] = 0u;
    __syncthreads();
    int bad = 0;
    for (int j = t; j < k; j += kThreads) {
        const int32_t i = ix[j];
        if (i < 0 || i >= vocab) {
            bad = 1;
        } else {
            const uint32_t bit = 1u << (i & 31);
            if (atomicOr(&bitmap[i >> 5], bit) & bit) bad = 1;
        }
    }
    bad = __syncthreads_or(bad);

    // the stored tokens' quantized logits and stored log-probabilities, loaded
    // now so that their latency hides behind the streaming pass (k <= 4 x 256)
    // (indices clamped into range so that every load is unconditional and all
    // of them are in flight together; slots past k or rows with bad ids are
    // masked where the values are used)
    int32_t ik[4];
    float lk[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int j = min(t + u * kThreads, k - 1);
        ik[u] = ix[j];
        lk[u] = lp[j];
    }
    EQ zraw[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) zraw[u] = row[min(max(ik[u], 0), static_cast<int32_t>(vocab - 1))];

    // ---- 2. stream the row: running max, lowest argmax, mass outside the stored tokens ----
    // The shift K is the wave's running maximum, the same in every lane: it
    // moves only when a ballot sees a new wave maximum (a few times per row),
    // and only then do the lanes holding that maximum record its first index
    // in their group (later equal values have higher indices). Lanes that are
    // idle in the last, partial step keep their own (K, wr) pair, which stays
    // self-consistent; the merge rescales every lane by exp(K - M).
    float m = -INFINITY;      // K
    float bestv = -INFINITY;  // value of this lane's record
    int best = INT32_MAX;     // index of this lane's record
    double wr = 0.0;          // mass outside the stored tokens, relative to K
    // one group of nz consecutive elements starting at i0, member bits in mbits
    // Every lane of the wave calls take the same number of times (nz = 0 for
    // an empty slot): the ballot and the wave maximum need all lanes.
    auto take = [&](int64_t i0, const float* z, int nz, uint32_t mbits) {
        float gm = -INFINITY;
        for (int j = 0; j < nz; ++j) gm = fmaxf(gm, z[j]);
        if (__any(gm > m)) {
            const float nk = wave_max(gm);
            if (m != -INFINITY) wr *= exp(static_cast<double>(m) - static_cast<double>(nk));
            m = nk;
            if (gm == nk) {
                int at = nz;  // first position of the new maximum (unrolled: z stays in registers)
#pragma unroll
                for (int j = 7; j >= 0; --j)
                    if (j < nz && z[j] == gm) at = j;
                best = static_cast<int>(i0) + at;
                bestv = nk;
            }
        }
        float s = 0.0f;
        if (mbits == 0u && nz == 8) {
            s = __builtin_amdgcn_exp2f((z[0] - m) * kLog2eF);
#pragma unroll
            for (int j = 1; j < 8; ++j) s += __builtin_amdgcn_exp2f((z[j] - m) * kLog2eF);
        } else {
            for (int j = 0; j < nz; ++j)
                if (!((mbits >> j) & 1u)) s += __builtin_amdgcn_exp2f((z[j] - m) * kLog2eF);
        }
        wr += static_cast<double>(s);
    };
    if constexpr (std::is_same<EQ, uint16_t>::value) {
        if (vec_ok) {
            // the same group update on packed pairs: the shifted values come
            // from pairs::shifted_tile, a new maximum shows as a positive one (integer
            // max of the bit patterns: positive floats order as positive ints,
            // negative ones and -0 are negative ints), and only then are the
            // values unpacked
            unsigned int slo, shi;
            asm volatile("v_mov_b32 %0, %1" : "=v"(slo) : "s"(0x00003f80u));  // bf16 pair (1, 0)
            asm volatile("v_mov_b32 %0, %1" : "=v"(shi) : "s"(0x3f800000u));  // bf16 pair (0, 1)
            stream_groups<KLD_TOPK_EVAL_U, 1, true>(row, vocab, t, [&](int64_t i0, const Raw8<EQ>& raw, bool ok) {
                float x[8];
                const u32x4 pr[1] = {raw.v};
                pairs::shifted_tile(raw.v, slo, shi, -m, x);
                int cmax = INT32_MIN;
                if (ok) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) cmax = max(cmax, __float_as_int(x[j]));
                }
                if (__any(cmax > 0)) {
                    const float gm = ok ? pairs::exact_max<1>(pr) : -INFINITY;
                    // the new shift, as a scalar (the same in every lane)
                    const float nk = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wave_max(gm))));
                    if (m != -INFINITY) wr *= exp(static_cast<double>(m) - static_cast<double>(nk));
                    m = nk;
                    if (ok && gm == nk) {
                        best = static_cast<int>(i0) + pairs::first_pair_slot<1>(pr, nk);
                        bestv = nk;
                    }
                    pairs::shifted_tile(raw.v, slo, shi, -m, x);
                }
                const uint32_t mbits = ok ? (bitmap[i0 >> 5] >> (i0 & 31)) & 0xffu : 0xffu;
                float sm = 0.0f;
                if (mbits == 0u) {
                    sm = __builtin_amdgcn_exp2f(x[0] * kLog2eF);
#pragma unroll
                    for (int j = 1; j < 8; ++j) sm += __builtin_amdgcn_exp2f(x[j] * kLog2eF);
                } else {
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        if (!((mbits >> j) & 1u)) sm += __builtin_amdgcn_exp2f(x[j] * kLog2eF);
                }
                wr += static_cast<double>(sm);
            });
        } else {
            for (int64_t c0 = 0; c0 < vocab; c0 += kThreads) {
                const int64_t i0 = c0 + t;
                const bool ok = i0 < vocab;
                const float z = ok ? widen(row[i0]) : 0.0f;
                take(i0, &z, ok ? 1 : 0, ok ? (bitmap[i0 >> 5] >> (i0 & 31)) & 1u : 0u);
            }
        }
    } else if (vec_ok) {
        stream_groups<KLD_TOPK_EVAL_U>(row, vocab, t, [&](int64_t i0, const float* z, bool ok) {
            take(i0, z, ok ? 8 : 0, ok ? (bitmap[i0 >> 5] >> (i0 & 31)) & 0xffu : 0u);
        });
    } else {
        for (int64_t c0 = 0; c0 < vocab; c0 += kThreads) {
            const int64_t i0 = c0 + t;
            const bool ok = i0 < vocab;
            const float z = ok ? widen(row[i0]) : 0.0f;
            take(i0, &z, ok ? 1 : 0, ok ? (bitmap[i0 >> 5] >> (i0 & 31)) & 1u : 0u);
        }
    }

    // ---- merge threads: row max and lowest argmax ----
    const float wm_ = wave_max(m);
    if ((t & 63) == 0) wmax[t >> 6] = wm_;
    __syncthreads();
    float M = wmax[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, wmax[w]);
    int cand = (bestv == M) ? best : INT32_MAX;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) cand = min(cand, __shfl_xor(cand, o));

    // ---- 3. per-thread float64 parts: rest mass (relative to M) and the stored tokens ----
    const double Md = static_cast<double>(M);
    double part[4];
    part[0] = (m == -INFINITY) ? 0.0 : wr * exp(static_cast<double>(m) - Md);  // mass outside the stored tokens
    part[1] = 0.0;  // sum_k exp(zq_k - M)
    part[2] = 0.0;  // sum_k p_k (log p_k - (zq_k - M))
    part[3] = 0.0;  // sum_k p_k
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        if (t + u * kThreads < k && !bad) {
            const double z = static_cast<double>(widen(zraw[u])) - Md;
            const double l = static_cast<double>(lk[u]);
            const double pk = exp(l);
            part[1] += exp(z);
            part[2] += pk * (l - z);
            part[3] += pk;
        }
    }
    // fixed butterfly inside each wave (lane 0's sums are used), then the waves in order
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) part[i] += __shfl_xor(part[i], o);
    }
    if ((t & 63) == 0) {
        widx[t >> 6] = cand;
#pragma unroll
        for (int i = 0; i < 4; ++i) wred[t >> 6][i] = part[i];
    }
    __syncthreads();
    double tot[4] = {0.0, 0.0, 0.0, 0.0};  // the same in every thread
    int iq = INT32_MAX;
    for (int w = 0; w < kWaves; ++w) {
        iq = min(iq, widx[w]);
#pragma unroll
        for (int i = 0; i < 4; ++i) tot[i] += wred[w][i];
    }
    // a rest mass too small for the stream's fp32 terms to hold (they are
    // shifted by the row maximum) is taken again, relative to its own maximum
    const int64_t n_rest = vocab - k;
    if (!bad && n_rest > 0 && tot[0] < static_cast<double>(n_rest) * kFarEval)
        tot[0] = sum_exp_below(
            row, vocab, vec_ok, Md, [&](float, int64_t i) { return !((bitmap[i >> 5] >> (i & 31)) & 1u); }, wmax,
            dres);
    if (t == 0) {
        const double wrest = tot[0];
        const double lnw = log(tot[1] + wrest);
        const double A = tot[2] + tot[3] * lnw;  // sum_k p_k (log p_k - log q_k)
        const double R = static_cast<double>(srest[r]);
        double kl = A;
        if (R > 0.0) kl += R * (log(R) - log(wrest) + lnw);
        const float klf = bad ? __builtin_nanf("") : static_cast<float>(kl);
        const int32_t ib = ix[0];
        const uint8_t mt = static_cast<uint8_t>(!bad && ib == iq);
        const int64_t gr = row_offset + r;
        const float nan = __builtin_nanf("");
        out.kld[gr] = klf;
        out.match[gr] = mt;
        out.argmax_b[gr] = ib;
        out.argmax_q[gr] = iq;
        out.lse_b[gr] = static_cast<double>(nan);
        out.lse_q[gr] = Md + lnw;
        if (out.topk_coef) {
            // The gradient's factors. A stored token's is q_j (P + R) - p_j; any
            // other token's q_j (P + R - R / Q_rest) is written as
            // exp(z_j - lse_rest) ((P + R) Q_rest - R), lse_rest = lse_q +
            // ln Q_rest the log of the rest's mass: the exponential is at most 1
            // (q_j <= Q_rest) and the factor lies in [-R, P + R], where R / Q_rest
            // alone overflows once the quant rest lies ~88 nats below its row's
            // maximum. A rest with no representable mass (Q_rest = 0 in float64:
            // KL_k is infinite when R > 0) keeps the plain form.
            const double call = tot[3] + R;
            double cout, lse_rest;
            if (wrest > 0.0) {
                cout = call * (wrest / (tot[1] + wrest)) - R;
                lse_rest = Md + log(wrest);
            } else {
                cout = R > 0.0 ? -static_cast<double>(INFINITY) : call;
                lse_rest = Md + lnw;
            }
            out.topk_coef[3 * gr] = bad ? static_cast<double>(nan) : call;
            out.topk_coef[3 * gr + 1] = bad ? static_cast<double>(nan) : cout;
            out.topk_coef[3 * gr + 2] = bad ? static_cast<double>(nan) : lse_rest;
        }
        out.logp_b[gr] = nan;
        out.logp_q[gr] = nan;
        out.dp[gr] = nan;
        out.tok_state[gr] = 0;
        if (out.kld_out) out.kld_out[r] = klf;
        if (out.match_out) out.match_out[r] = mt;
        if (out.argmax_b_out) out.argmax_b_out[r] = ib;
        if (out.argmax_q_out) out.argmax_q_out[r] = iq;
    }
}


// ------------------------------------------------------------------ grad ---

#ifndef KLD_TOPK_GRAD_G_F32
#define KLD_TOPK_GRAD_G_F32 2  // groups of 2048 elements per workgroup, float32 output
#endif
#ifndef KLD_TOPK_GRAD_G_BF16
#define KLD_TOPK_GRAD_G_BF16 4  // groups of 2048 elements per workgroup, bfloat16 output
#endif

// Output layout per group of 2048 elements. float32: wave w covers
// [512 w, 512 w + 512), lane l its elements 4 l .. 4 l + 3 and 256 + 4 l ..
// 256 + 4 l + 3, so each 16-byte store instruction of a wave writes one
// contiguous 1 KiB; bfloat16: thread t owns 8 contiguous elements at 8 t.
template <class EG>
struct GradLayout;
template <>
struct GradLayout<float> {
    static constexpr int kGroups = KLD_TOPK_GRAD_G_F32;
    static constexpr int kRun = 4;  // two runs of 4 elements, 256 apart
    __device__ static int64_t offset(int t) { return static_cast<int64_t>(t >> 6) * 512 + 4 * (t & 63); }
};
template <>
struct GradLayout<uint16_t> {
    static constexpr int kGroups = KLD_TOPK_GRAD_G_BF16;
    static constexpr int kRun = 8;  // one run of 8 elements
    __device__ static int64_t offset(int t) { return static_cast<int64_t>(t) * 8; }
};
constexpr int64_t kXcds = 8;  // accelerator complexes (each with its own L2) on gfx950

template <class EG>
constexpr int64_t grad_chunk() {
    return static_cast<int64_t>(GradLayout<EG>::kGroups) * kThreads * 8;
}

// kRun elements at p (kRun = 4 or 8), zero-filled when !ok.
template <int kRun>
__device__ __forceinline__ void load_run(const uint16_t* p, bool ok, float* z) {
    if constexpr (kRun == 4) {
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 a = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p)) : u32x2{0u, 0u};
        z[0] = __uint_as_float(a[0] << 16); z[1] = __uint_as_float(a[0] & 0xffff0000u);
        z[2] = __uint_as_float(a[1] << 16); z[3] = __uint_as_float(a[1] & 0xffff0000u);
    } else {
        const u32x4 a = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            z[2 * j] = __uint_as_float(a[j] << 16);
            z[2 * j + 1] = __uint_as_float(a[j] & 0xffff0000u);
        }
    }
}
template <int kRun>
__device__ __forceinline__ void load_run(const float* p, bool ok, float* z) {
#pragma unroll
    for (int h = 0; h < kRun / 4; ++h) {
        const f32x4 a = ok ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4 * h))
                           : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) z[4 * h + j] = a[j];
    }
}

__device__ __forceinline__ unsigned int to_bf16_rne(float x) {
    const unsigned int u = __float_as_uint(x);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// kRun outputs at p.
__device__ __forceinline__ void store_run(float* p, const float* g) {
    __builtin_nontemporal_store(f32x4{g[0], g[1], g[2], g[3]}, reinterpret_cast<f32x4*>(p));
}
__device__ __forceinline__ void store_run(uint16_t* p, const float* g) {
    u32x4 v;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = to_bf16_rne(g[2 * j]) | (to_bf16_rne(g[2 * j + 1]) << 16);
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void store_one(float* p, float g) { *p = g; }
__device__ __forceinline__ void store_one(uint16_t* p, float g) { *p = static_cast<uint16_t>(to_bf16_rne(g)); }

// Gradient of KL_k (stored form fixed) with respect to the quantized logits:
//   g_j = w (q_j (P + R) - [j stored] p_j - [j not stored] R q_j / Q_rest),
// P = sum of the stored probabilities, R the stored rest mass, q from the
// row's float64 log-normaliser; the evaluation kernel saved lse_q and, per
// row, P + R, (P + R) Q_rest - R and lse_rest = lse_q + ln Q_rest (NaN for a
// row with bad ids): a token outside the stored ones gets
// w exp(z_j - lse_rest) ((P + R) Q_rest - R), the same value with both
// factors bounded however far below its maximum the quant row's rest lies.
// Each workgroup takes one chunk of one row. The quant loads go out first;
// meanwhile the stored ids that fall in the chunk are marked in an LDS bitmap
// and each one's p_j is placed at its rank among them (prefix popcounts of
// the bitmap), so that the thread streaming a stored token finds its p_j
// without a search and every output is written once, in whole vectors. A row
// with ids outside [0, vocab) or repeated has NaN factors and is written as
// NaN; each chunk also checks the ids it sees, and never uses a bad one.
template <class EQ, class EG>
__global__ void __launch_bounds__(kThreads)
    topk_grad_kernel(const EQ* __restrict__ quant, const int32_t* __restrict__ sidx, const float* __restrict__ slogp,
                     int64_t vocab, int k, int chunks_per_row, int vec_ok, int64_t row_offset,
                     const double* __restrict__ lse_q, const double* __restrict__ coef, float scale,
                     EG* __restrict__ grad) {
    using L = GradLayout<EG>;
    constexpr int64_t kChunk = grad_chunk<EG>();
    constexpr int kWords = static_cast<int>(kChunk / 32);
    static_assert(kWords <= kThreads, "one bitmap word per thread in the rank scan");
    constexpr int kRun = L::kRun;
    constexpr int kIdsPerThread = kMaxK / kThreads;
    __shared__ uint32_t bitmap[kWords];
    __shared__ uint32_t rank0[kWords];  // stored tokens of the chunk before each bitmap word
    __shared__ double pm[kMaxK];        // p_j of the chunk's stored tokens, in index order
    __shared__ uint32_t wsum[kWaves];
    const int t = threadIdx.x;
    // Workgroup ids are dealt to the 8 XCDs in turn; renumber them so that
    // each XCD takes one contiguous run of chunks (ids past the largest
    // multiple of 8 keep their number). The chunks of a row then share one L2,
    // which serves the row's stored ids to all of them after the first.
    const int64_t nwg = gridDim.x, per_xcd = nwg / kXcds;
    const int64_t hw = blockIdx.x;
    const int64_t bid = hw < per_xcd * kXcds ? (hw % kXcds) * per_xcd + hw / kXcds : hw;
    const int64_t r = bid / chunks_per_row;
    const int64_t c0 = (bid - r * chunks_per_row) * kChunk;
    const int64_t c1 = min(vocab, c0 + kChunk);
    const EQ* row = quant + r * vocab;
    EG* gr = grad + r * vocab;
    const int32_t* ix = sidx + r * k;
    const float* lp = slogp + r * k;

    // quant loads first: nothing below changes which elements they read
    float z[L::kGroups][8];
    if (vec_ok) {
#pragma unroll
        for (int u = 0; u < L::kGroups; ++u) {
            const int64_t i = c0 + u * 2048 + L::offset(t);
            load_run<kRun>(row + i, i < c1, z[u]);
            if constexpr (kRun == 4) load_run<kRun>(row + i + 256, i + 256 < c1, z[u] + 4);
        }
    }
    for (int w = t; w < kWords; w += kThreads) bitmap[w] = 0u;
    __syncthreads();
    int bad = 0;
    int32_t ik[kIdsPerThread];
#pragma unroll
    for (int u = 0; u < kIdsPerThread; ++u) {
        const int j = t + u * kThreads;
        ik[u] = -1;
        if (j < k) {
            const int32_t i = ix[j];
            if (i < 0 || i >= vocab) {
                bad = 1;
            } else if (i >= c0 && i < c1) {
                const int o = static_cast<int>(i - c0);
                const uint32_t bit = 1u << (o & 31);
                if (atomicOr(&bitmap[o >> 5], bit) & bit) bad = 1;
                ik[u] = o;
            }
        }
    }
    bad = __syncthreads_or(bad);
    uint32_t n_in;
    const uint32_t ex = block_scan2(t < kWords ? static_cast<uint32_t>(__popc(bitmap[t])) : 0u, wsum, n_in);
    if (t < kWords) rank0[t] = ex;
    __syncthreads();
    // rank of chunk offset o among the chunk's stored tokens (o must be one)
    auto rank = [&](int o) { return rank0[o >> 5] + __popc(bitmap[o >> 5] & ((1u << (o & 31)) - 1u)); };
    if (!bad) {
#pragma unroll
        for (int u = 0; u < kIdsPerThread; ++u)
            if (ik[u] >= 0) pm[rank(ik[u])] = exp(static_cast<double>(lp[t + u * kThreads]));
    }
    __syncthreads();

    const double L_ = lse_q[row_offset + r];
    const double call = bad ? static_cast<double>(__builtin_nanf("")) : coef[3 * (row_offset + r)];
    const double cout = bad ? static_cast<double>(__builtin_nanf("")) : coef[3 * (row_offset + r) + 1];
    const double Lr = bad ? static_cast<double>(__builtin_nanf("")) : coef[3 * (row_offset + r) + 2];
    const double w = static_cast<double>(scale);
    const float f_out = static_cast<float>(w * cout);
    // exp(x - L) for a double L as exp2((x - s) log2(e) - c), s = L rounded to float
    const float s = static_cast<float>(L_);
    const float c = static_cast<float>((L_ - static_cast<double>(s)) * 1.4426950408889634);
    const float sr = static_cast<float>(Lr);
    const float cr = static_cast<float>((Lr - static_cast<double>(sr)) * 1.4426950408889634);
    auto prob = [&](float x) { return __builtin_amdgcn_exp2f(fmaf(x - s, kLog2eF, -c)); };
    auto prob_rest = [&](float x) { return __builtin_amdgcn_exp2f(fmaf(x - sr, kLog2eF, -cr)); };
    auto stored = [&](float q, int o) { return static_cast<float>(w * (static_cast<double>(q) * call - pm[rank(o)])); };
    // a NaN row is written whole by the stream, and pm was not filled
    const uint32_t live = (call == call) ? 0xffu : 0u;

    if (vec_ok) {
#pragma unroll
        for (int u = 0; u < L::kGroups; ++u) {
            const int64_t i = c0 + u * 2048 + L::offset(t);
            const int o = static_cast<int>(i - c0);
#pragma unroll
            for (int h = 0; h < 8 / kRun; ++h) {
                const int oh = o + h * 256;
                if (i + h * 256 < c1) {
                    float g[kRun];
#pragma unroll
                    for (int j = 0; j < kRun; ++j) g[j] = prob_rest(z[u][h * kRun + j]) * f_out;
                    const uint32_t m = (bitmap[oh >> 5] >> (oh & 31)) & ((1u << kRun) - 1u) & live;
                    if (m) {  // rare: a stored token in this run
#pragma unroll
                        for (int j = 0; j < kRun; ++j)
                            if ((m >> j) & 1u) g[j] = stored(prob(z[u][h * kRun + j]), oh + j);
                    }
                    store_run(gr + i + h * 256, g);
                }
            }
        }
    } else {
        for (int64_t i = c0 + t; i < c1; i += kThreads) {
            const int o = static_cast<int>(i - c0);
            const float zi = widen(row[i]);
            float g = prob_rest(zi) * f_out;
            if ((bitmap[o >> 5] >> (o & 31)) & live & 1u) g = stored(prob(zi), o);
            store_one(gr + i, g);
        }
    }
}

}  // namespace

int topk_max_k() { return kMaxK; }

hipError_t launch_topk_compress(int base_type, const void* base, int64_t vocab, int64_t n_rows, int k,
                                int32_t* idx_out, float* logp_out, float* rest_out, hipStream_t stream) {
    const bool vec_ok = vocab % 8 == 0 && reinterpret_cast<uintptr_t>(base) % 16 == 0;
    const size_t esz = base_type == kF32 ? 4 : 2;
    const int64_t per = max_blocks_per_launch(kThreads);
    for (int64_t done = 0; done < n_rows; done += per) {
        const int64_t n = n_rows - done < per ? n_rows - done : per;
        const void* b = static_cast<const char*>(base) + static_cast<size_t>(done) * vocab * esz;
        const bool large = k > kThreads;
        if (base_type == kF32 && !large)
            hipLaunchKernelGGL((topk_compress_kernel<float, false>), dim3(static_cast<unsigned>(n)), dim3(kThreads), 0,
                               stream, static_cast<const float*>(b), vocab, k, vec_ok ? 1 : 0, idx_out + done * k,
                               logp_out + done * k, rest_out + done);
        else if (base_type == kF32)
            hipLaunchKernelGGL((topk_compress_kernel<float, true>), dim3(static_cast<unsigned>(n)), dim3(kThreads), 0,
                               stream, static_cast<const float*>(b), vocab, k, vec_ok ? 1 : 0, idx_out + done * k,
                               logp_out + done * k, rest_out + done);
        else if (!large)
            hipLaunchKernelGGL((topk_compress_kernel<uint16_t, false>), dim3(static_cast<unsigned>(n)), dim3(kThreads),
                               0, stream, static_cast<const uint16_t*>(b), vocab, k, vec_ok ? 1 : 0,
                               idx_out + done * k, logp_out + done * k, rest_out + done);
        else
            hipLaunchKernelGGL((topk_compress_kernel<uint16_t, true>), dim3(static_cast<unsigned>(n)), dim3(kThreads),
                               0, stream, static_cast<const uint16_t*>(b), vocab, k, vec_ok ? 1 : 0,
                               idx_out + done * k, logp_out + done * k, rest_out + done);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_topk_eval(int quant_type, const int32_t* idx, const float* logp, const float* rest, int k,
                            const void* quant, int64_t vocab, int64_t n_rows, int64_t row_offset, const RowOut& out,
                            hipStream_t stream) {
    const bool vec_ok = vocab % 8 == 0 && reinterpret_cast<uintptr_t>(quant) % 16 == 0;
    const size_t lds = static_cast<size_t>((vocab + 31) / 32) * sizeof(uint32_t);
    const size_t esz = quant_type == kF32 ? 4 : 2;
    if (lds > 65536) {  // large token maps: raise the kernel's dynamic LDS limit first
        hipError_t e = quant_type == kF32
                           ? hipFuncSetAttribute(reinterpret_cast<const void*>(topk_eval_kernel<float>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds))
                           : hipFuncSetAttribute(reinterpret_cast<const void*>(topk_eval_kernel<uint16_t>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (e != hipSuccess) return e;
    }
    const int64_t per = max_blocks_per_launch(kThreads);
    for (int64_t done = 0; done < n_rows; done += per) {
        const int64_t n = n_rows - done < per ? n_rows - done : per;
        RowOut o = out;
        if (o.kld_out) o.kld_out += done;
        if (o.match_out) o.match_out += done;
        if (o.argmax_b_out) o.argmax_b_out += done;
        if (o.argmax_q_out) o.argmax_q_out += done;
        const void* q = static_cast<const char*>(quant) + static_cast<size_t>(done) * vocab * esz;
        if (quant_type == kF32)
            hipLaunchKernelGGL(topk_eval_kernel<float>, dim3(static_cast<unsigned>(n)), dim3(kThreads), lds, stream,
                               static_cast<const float*>(q), idx + done * k, logp + done * k, rest + done, vocab, k,
                               vec_ok ? 1 : 0, row_offset + done, o);
        else
            hipLaunchKernelGGL(topk_eval_kernel<uint16_t>, dim3(static_cast<unsigned>(n)), dim3(kThreads), lds,
                               stream, static_cast<const uint16_t*>(q), idx + done * k, logp + done * k, rest + done,
                               vocab, k, vec_ok ? 1 : 0, row_offset + done, o);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}


namespace {
// One element type pair, launched in row pieces of at most
// max_blocks_per_launch workgroups.
template <class EQ, class EG>
hipError_t topk_grad_launch(const int32_t* idx, const float* logp, int k, const EQ* quant, int64_t vocab,
                            int64_t n_rows, int64_t row_offset, const double* lse_q, const double* coef, float scale,
                            EG* grad, hipStream_t stream) {
    const int64_t cpr = (vocab + grad_chunk<EG>() - 1) / grad_chunk<EG>();
    const bool vec_ok = vocab % 8 == 0 && reinterpret_cast<uintptr_t>(quant) % 16 == 0 &&
                        reinterpret_cast<uintptr_t>(grad) % 16 == 0;
    const int64_t rows_per_launch = max_blocks_per_launch(kThreads) / cpr;
    for (int64_t done = 0; done < n_rows; done += rows_per_launch) {
        const int64_t n = n_rows - done < rows_per_launch ? n_rows - done : rows_per_launch;
        hipLaunchKernelGGL((topk_grad_kernel<EQ, EG>), dim3(static_cast<unsigned>(n * cpr)), dim3(kThreads), 0,
                           stream, quant + done * vocab, idx + done * k, logp + done * k, vocab, k,
                           static_cast<int>(cpr), vec_ok ? 1 : 0, row_offset + done, lse_q, coef, scale,
                           grad + done * vocab);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}
}  // namespace

hipError_t launch_topk_grad(int quant_type, int grad_type, const int32_t* idx, const float* logp, int k,
                            const void* quant, int64_t vocab, int64_t n_rows, int64_t row_offset,
                            const double* lse_q, const double* coef, float scale, void* grad, hipStream_t stream) {
    if (quant_type == kF32)
        return grad_type == kF32
                   ? topk_grad_launch(idx, logp, k, static_cast<const float*>(quant), vocab, n_rows, row_offset,
                                      lse_q, coef, scale, static_cast<float*>(grad), stream)
                   : topk_grad_launch(idx, logp, k, static_cast<const float*>(quant), vocab, n_rows, row_offset,
                                      lse_q, coef, scale, static_cast<uint16_t*>(grad), stream);
    return grad_type == kF32
               ? topk_grad_launch(idx, logp, k, static_cast<const uint16_t*>(quant), vocab, n_rows, row_offset,
                                  lse_q, coef, scale, static_cast<float*>(grad), stream)
               : topk_grad_launch(idx, logp, k, static_cast<const uint16_t*>(quant), vocab, n_rows, row_offset,
                                  lse_q, coef, scale, static_cast<uint16_t*>(grad), stream);
}

}  // namespace kldk
