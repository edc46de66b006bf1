// Fused per-row kernel: KL(P_base || Q_quant), both argmaxes and both
// log-normalisers of one pair of logit rows, in a single pass over HBM.
//
// What is computed follows the GSQ-RCO model card ("How it was made" step 5:
// KL of the quantized model's output from the BF16 model's, over the full
// vocabulary) and the Qwen3.6 27B quantization benchmark ("Understand KLD and
// Same Top P": drift of the confidence distribution, and whether both models
// pick the same top token). Argmax ties go to the lowest index.
//
// Work decomposition (gfx950, wave64): one workgroup of NW waves per row pair.
// The row is cut into wave-tiles of 512 elements; wave w takes wave-tiles
// w, w + NW, w + 2 NW, ...; inside a wave-tile each lane owns 8 elements, so
// every load instruction of the wave covers one contiguous span (1 KiB for
// 16-byte loads, 512 B for the 8-byte bf16 loads of a mixed-type pair). Lanes see their
// elements in ascending index order. Elements past the last full wave-tile
// (and whole rows whose shape or alignment rules out 16-byte loads) go
// through a predicated element-wise path with the same arithmetic.
//
// Numerics. Each wave keeps a wave-uniform shift per row equal to the exact
// running maximum of that row's logits (Kb, Kq). For every element, in fp32,
//   tb = (zb - Kb) log2(e),  tq = (zq - Kq) log2(e),  v = tb - tq
//   w  = 2^tb,  e = 2^tq,  t = e - w
//   W += w,  C += t,  P += t log2(e) + w v
// so that W = sum exp(zb - Kb), W + C = sum exp(zq - Kq) and, with
// x = C / W, KL = ln2 P / W + (log1p(x) - x) (evaluated in float64 once per
// row). P collects per-token terms ~ w v^2 ln2 / 2 that are never large, so
// fp32 rounding of the accumulators scales with the divergence itself, not
// with the mean log-ratio; the error of C enters only through
// log1p(x) - x ~ -x^2 / 2. v is formed from the very arguments handed to the
// exponentials, so the result is the exact divergence of logits perturbed by
// the rounding of (z - K) log2(e) (relative 2^-24), an error that is second
// order in the per-token terms. At the token that is the maximum of both rows
// tb = tq = 0 exactly, so w = e = 1 exactly and it adds nothing to C or P. A
// shift moves only when a chunk holds a new maximum (a wave ballot); then the
// accumulated terms are re-expressed in the new shifts (see rescale_factors)
// and the same operator merges the waves of a workgroup. The argmax is found
// without per-element index tracking: when a chunk moves the wave's running
// maximum, the lanes holding the new maximum record the index of its first
// occurrence in their part of the chunk (the chunk is still in registers);
// the row's argmax is the lowest recorded index among the lanes whose record
// equals the row maximum.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "kld_bf16_pairs.h"
#include "kld_kernels.h"

namespace kldk {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kWaveTile = 512;  // elements per wave-tile (64 lanes x 8)
constexpr int kTailPerLane = 4;  // elements per lane per predicated chunk
// Build-time constants: partial sums per lane, the prefetch ring of the
// bf16-pair path and the number of waves per SIMD its register allocation
// must leave room for. The launch shape itself (waves per row) is picked per
// handle in launch_rows.
#ifndef KLD_SLOTS
#define KLD_SLOTS 8
#endif
#ifndef KLD_BB_MIN_WAVES
#define KLD_BB_MIN_WAVES 1
#endif
#ifndef KLD_DEPTH
#define KLD_DEPTH 4  // register sets in the prefetch ring (chunks in flight + 1)
#endif
#ifndef KLD_BB_UNROLL
#define KLD_BB_UNROLL 1  // wave-tiles per chunk, both rows bf16
#endif
constexpr int kSlots = KLD_SLOTS;  // independent partial sums per lane

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct TF32 {
    using elem = float;
};
struct TBF16 {
    using elem = uint16_t;
};

using pairs::bf16_hi;
using pairs::bf16_lo;
using pairs::exact_max;
using pairs::first_pair_slot;
using pairs::shifted_tile;

__device__ __forceinline__ float load_elem(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_elem(const uint16_t* p, int64_t i) {
    return __uint_as_float(static_cast<unsigned int>(p[i]) << 16);
}

// Position of tile element j of `lane` inside a wave-tile. With both rows in
// bf16 a lane owns 8 consecutive elements (one 16-byte load per row);
// otherwise it owns [4 lane, 4 lane + 4) and [256 + 4 lane, 256 + 4 lane + 4).
template <bool kContig8>
__device__ __forceinline__ int tile_pos(int lane, int j) {
    if (kContig8) return lane * 8 + j;
    return (j < 4) ? lane * 4 + j : 256 + lane * 4 + (j - 4);
}

template <class T, bool kContig8>
struct Tile;

template <>
struct Tile<TBF16, true> {
    struct Raw {
        u32x4 v;
    };
    static __device__ __forceinline__ Raw load(const uint16_t* wt, int lane) {
        Raw r;
        r.v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wt) + static_cast<unsigned int>(lane));
        return r;
    }
    static __device__ __forceinline__ void unpack(const Raw& r, float z[8]) {
        z[0] = bf16_lo(r.v.x); z[1] = bf16_hi(r.v.x);
        z[2] = bf16_lo(r.v.y); z[3] = bf16_hi(r.v.y);
        z[4] = bf16_lo(r.v.z); z[5] = bf16_hi(r.v.z);
        z[6] = bf16_lo(r.v.w); z[7] = bf16_hi(r.v.w);
    }
};

template <>
struct Tile<TBF16, false> {
    struct Raw {
        u32x2 a, b;
    };
    static __device__ __forceinline__ Raw load(const uint16_t* wt, int lane) {
        Raw r;
        r.a = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(wt) + static_cast<unsigned int>(lane));
        r.b = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(wt + 256) + static_cast<unsigned int>(lane));
        return r;
    }
    static __device__ __forceinline__ void unpack(const Raw& r, float z[8]) {
        z[0] = bf16_lo(r.a.x); z[1] = bf16_hi(r.a.x);
        z[2] = bf16_lo(r.a.y); z[3] = bf16_hi(r.a.y);
        z[4] = bf16_lo(r.b.x); z[5] = bf16_hi(r.b.x);
        z[6] = bf16_lo(r.b.y); z[7] = bf16_hi(r.b.y);
    }
};

template <>
struct Tile<TF32, false> {
    struct Raw {
        f32x4 a, b;
    };
    static __device__ __forceinline__ Raw load(const float* wt, int lane) {
        Raw r;
        r.a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(wt) + static_cast<unsigned int>(lane));
        r.b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(wt + 256) + static_cast<unsigned int>(lane));
        return r;
    }
    static __device__ __forceinline__ void unpack(const Raw& r, float z[8]) {
        z[0] = r.a.x; z[1] = r.a.y; z[2] = r.a.z; z[3] = r.a.w;
        z[4] = r.b.x; z[5] = r.b.y; z[6] = r.b.z; z[7] = r.b.w;
    }
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float uniform(float v) {
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

// Per-lane partial sums, all relative to the wave's current shifts. A lane
// sees V / 64 elements of a row in the one-wave shape (V / 256 with four
// waves), so its fp32 slots are folded every kFoldChunks chunks into
// second-level sums W2, C2, P2 held in float64: an fp32 sum then never takes
// more than a few dozen terms. (Summing many equal terms -- tied logits, or a
// row flat but for a few tokens -- rounds the same way each time, so an fp32
// sum's error grows with its count, not its square root; in fp32 the second
// level too drifts past the normaliser's bound from V ~ 2^24 on such rows.)
// The second level lives in LDS, three doubles per lane, touched only at a
// fold or a rescale, so it costs no registers in the streaming loop.
struct Acc {
    float W[kSlots], C[kSlots], P[kSlots];
};
constexpr int kFoldChunks = 32;

__device__ __forceinline__ float slot_sum(const float (&a)[kSlots]) {
    static_assert(kSlots == 8, "fixed pairwise order");
    return ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
}

// l2: this lane's second-level sums W2, C2, P2 (LDS)
__device__ __forceinline__ void fold_slots(Acc& a, double* l2) {
    atomicAdd(&l2[0], static_cast<double>(slot_sum(a.W)));
    atomicAdd(&l2[1], static_cast<double>(slot_sum(a.C)));
    atomicAdd(&l2[2], static_cast<double>(slot_sum(a.P)));
#pragma unroll
    for (int s = 0; s < kSlots; ++s) {
        a.W[s] = 0.0f;
        a.C[s] = 0.0f;
        a.P[s] = 0.0f;
    }
}

// Factors that re-express a state taken with shifts (Kb, Kq) in shifts
// (nb, nq), nb >= Kb, nq >= Kq (db = nb - Kb, dq = nq - Kq, d = db - dq):
//   W' = e^-db W
//   C' = e^-dq C + e^-db expm1(d) W
//   P' = e^-db P + log2(e) (e^-db expm1(d) C + e^-db (expm1(d) - d) W)
// Each coefficient is formed as one bounded quantity (e^-db e^d is taken as
// e^-dq), so shifts that are thousands of nats apart give 0, never 0 * inf.
// Evaluated in float64: the factors are uniform per wave and needed only when
// a maximum moves (a few times per row).
struct Rescale {
    float fw, fcc, fcw, fpc, fpw;
};

__device__ __forceinline__ Rescale rescale_factors(float Kb, float Kq, float nb, float nq) {
    constexpr double kL = 1.4426950408889634;  // log2(e): P is kept in log2 units
    const double db = static_cast<double>(nb) - static_cast<double>(Kb);  // >= 0
    const double dq = static_cast<double>(nq) - static_cast<double>(Kq);  // >= 0
    const double d = db - dq;
    const double r = exp(-db);
    const double rq = exp(-dq);
    double cw, pw;
    if (fabs(d) < 0.5) {
        const double em1 = expm1(d);  // accurate near 0, where e^d - 1 and e^d - 1 - d are small
        cw = r * em1;
        pw = r * (em1 - d);
    } else {
        cw = rq - r;       // = e^-db (e^d - 1)
        pw = cw - d * r;   // = e^-db (e^d - 1 - d)
    }
    Rescale f;
    f.fw = static_cast<float>(r);
    f.fcc = static_cast<float>(rq);
    f.fcw = static_cast<float>(cw);
    f.fpc = static_cast<float>(kL * cw);
    f.fpw = static_cast<float>(kL * pw);
    return f;
}

__device__ __forceinline__ void apply_rescale(float& W, float& C, float& P, const Rescale& f) {
    const float w = W, c = C;
    P = fmaf(f.fw, P, fmaf(f.fpc, c, f.fpw * w));
    C = fmaf(f.fcc, c, f.fcw * w);
    W = f.fw * w;
}

// Row-level running state of one lane.
struct LaneState {
    float Kb, Kq;        // wave-uniform shifts: exact running maxima of the wave's elements
    float bestb, bestq;  // lane maxima recorded when they equalled the wave's running maximum
    int idxb, idxq;      // element index of the first such occurrence (INT32_MAX: none)
    float carried;       // mass moved between W and C by rescales (|fcw| W each), scaled
                         // by every later rescale as C and P are: its rounding's reach now
    Acc acc;
    double* l2;          // this lane's second-level sums W2, C2, P2 (LDS)
};

// A rescale: the slots first join the second level (and restart from zero),
// so only the three float64 sums are re-expressed in the new shifts. The mass
// it moves between W and C, |fcw| W, is added to `carried`, whose earlier
// content is scaled as C and P are.
__device__ __forceinline__ void fold_and_rescale(LaneState& st, const Rescale& f) {
    double* const l2 = st.l2;
    const double w = l2[0] + static_cast<double>(slot_sum(st.acc.W));
    const double c = l2[1] + static_cast<double>(slot_sum(st.acc.C));
    const double p = l2[2] + static_cast<double>(slot_sum(st.acc.P));
#pragma unroll
    for (int s = 0; s < kSlots; ++s) {
        st.acc.W[s] = 0.0f;
        st.acc.C[s] = 0.0f;
        st.acc.P[s] = 0.0f;
    }
    st.carried = fmaf(fabsf(f.fcw), static_cast<float>(w), st.carried * fmaxf(f.fw, f.fcc));
    l2[2] = fma(static_cast<double>(f.fw), p, fma(static_cast<double>(f.fpc), c, static_cast<double>(f.fpw) * w));
    l2[1] = fma(static_cast<double>(f.fcc), c, static_cast<double>(f.fcw) * w);
    l2[0] = static_cast<double>(f.fw) * w;
}

// First slot of z[] (in slot order, which is index order) holding m.
template <int N>
__device__ __forceinline__ int first_slot(const float (&z)[N], float m) {
    int at = N;
#pragma unroll
    for (int i = N - 1; i >= 0; --i) at = (z[i] == m) ? i : at;
    return at;
}

// Process N elements per lane (one chunk); slot i holds element index_of(i),
// increasing with i. kMasked: elements may be invalid (zb = zq = -inf there)
// and contribute nothing.
template <int N, bool kMasked, int kSlot0 = 0, class IndexOf>
__device__ __forceinline__ void chunk_update(const float (&zb)[N], const float (&zq)[N], LaneState& st,
                                             IndexOf index_of) {
    float cb = zb[0], cq = zq[0];
#pragma unroll
    for (int i = 1; i < N; ++i) {
        cb = fmaxf(cb, zb[i]);
        cq = fmaxf(cq, zq[i]);
    }
    if (__any((cb > st.Kb) || (cq > st.Kq))) {
        const float nb = uniform(fmaxf(wave_max(cb), st.Kb));
        const float nq = uniform(fmaxf(wave_max(cq), st.Kq));
        if (st.Kb != -INFINITY) {  // otherwise nothing has been accumulated yet
            fold_and_rescale(st, rescale_factors(st.Kb, st.Kq, nb, nq));
        }
        st.Kb = nb;
        st.Kq = nq;
        // Argmax records. A lane's first occurrence of the final row maximum
        // lies in a chunk that raised the wave's running maximum (or tied the
        // new value in that same chunk): a later chunk of this wave only holds
        // higher indices. So records are only taken here, when a maximum
        // moves, by the lanes whose chunk holds the new wave maximum, with the
        // exact element index; the strict > keeps a lane's earliest one.
        if (cb == nb && cb > st.bestb) {
            st.bestb = cb;
            st.idxb = index_of(first_slot<N>(zb, nb));
        }
        if (cq == nq && cq > st.bestq) {
            st.bestq = cq;
            st.idxq = index_of(first_slot<N>(zq, nq));
        }
    }
    if (kMasked && st.Kb == -INFINITY) return;  // no valid element in this wave yet
    const float Kb = st.Kb, Kq = st.Kq;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float tb = (zb[i] - Kb) * kLog2e;
        const float tq = (zq[i] - Kq) * kLog2e;
        const float w = __builtin_amdgcn_exp2f(tb);
        const float e = __builtin_amdgcn_exp2f(tq);
        float v = tb - tq;
        if (kMasked) v = (zb[i] == -INFINITY) ? 0.0f : v;
        const float t = e - w;
        const int s = (i + kSlot0) % kSlots;
        st.acc.W[s] += w;
        st.acc.C[s] += t;
        st.acc.P[s] = fmaf(w, v, fmaf(t, kLog2e, st.acc.P[s]));
    }
}

// Both rows in bf16, 8 consecutive elements per lane per wave-tile: the same
// update as chunk_update, with the shifted values formed straight from the
// packed pairs. v_dot2_f32_bf16(pair, (1, 0), -K) = lo - K and
// v_dot2_f32_bf16(pair, (0, 1), -K) = hi - K: the products by 1 and 0 are
// exact, so the result equals the fp32 subtraction whenever that is exact
// (always at or near the running maximum) and differs from it by the
// direction of rounding otherwise, which is immaterial because every later
// term uses this same value. It keeps x = 0 exactly at z = K and x > 0 exactly
// when z > K, so a new maximum shows as max(x) > 0; only then are the exact
// values unpacked (for the new shift and the argmax records) and x formed
// again with the new shift. The two selectors arrive as kernel arguments and
// are held in vector registers.

template <int U>
__device__ __forceinline__ void shifted_pairs(const u32x4 (&r)[U], float negk, unsigned int slo, unsigned int shi,
                                              float (&x)[U * 8]) {
#pragma unroll
    for (int u = 0; u < U; ++u) shifted_tile(r[u], slo, shi, negk, &x[u * 8]);
}

template <int U, class IndexOf>
__device__ __forceinline__ void chunk_update_bf16_pairs(const u32x4 (&rb)[U], const u32x4 (&rq)[U], LaneState& st,
                                                        IndexOf index_of, unsigned int slo, unsigned int shi) {
    constexpr int N = U * 8;
    float xb[N], xq[N];
    shifted_pairs<U>(rb, -st.Kb, slo, shi, xb);
    shifted_pairs<U>(rq, -st.Kq, slo, shi, xq);
    // Is any shifted value positive (a new maximum)? On the bit patterns:
    // positive floats order like positive ints and every negative float
    // (and -0) is a negative int, so the integer maximum is > 0 exactly when
    // some value is > 0 -- and integer max needs no NaN canonicalization.
    int cmax = __float_as_int(xb[0]);
#pragma unroll
    for (int i = 1; i < N; ++i) cmax = max(cmax, __float_as_int(xb[i]));
#pragma unroll
    for (int i = 0; i < N; ++i) cmax = max(cmax, __float_as_int(xq[i]));
    if (__any(cmax > 0)) {
        const float zb = exact_max<U>(rb), zq = exact_max<U>(rq);
        const float nb = uniform(fmaxf(wave_max(zb), st.Kb));
        const float nq = uniform(fmaxf(wave_max(zq), st.Kq));
        if (st.Kb != -INFINITY) {
            fold_and_rescale(st, rescale_factors(st.Kb, st.Kq, nb, nq));
        }
        st.Kb = nb;
        st.Kq = nq;
        if (zb == nb && zb > st.bestb) {  // argmax records, as in chunk_update
            st.bestb = zb;
            st.idxb = index_of(first_pair_slot<U>(rb, nb));
        }
        if (zq == nq && zq > st.bestq) {
            st.bestq = zq;
            st.idxq = index_of(first_pair_slot<U>(rq, nq));
        }
        shifted_pairs<U>(rb, -nb, slo, shi, xb);
        shifted_pairs<U>(rq, -nq, slo, shi, xq);
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float tb = xb[i] * kLog2e;
        const float tq = xq[i] * kLog2e;
        const float w = __builtin_amdgcn_exp2f(tb);
        const float e = __builtin_amdgcn_exp2f(tq);
        const float v = tb - tq;
        const float t = e - w;
        const int s = i % kSlots;
        st.acc.W[s] += w;
        st.acc.C[s] += t;
        st.acc.P[s] = fmaf(w, v, fmaf(t, kLog2e, st.acc.P[s]));
    }
}

// Per-wave state as exchanged through LDS.
struct WaveState {
    float Kb, Kq, W, C, P, carried;
};

// Merge the per-wave states in wave order into shifts (Tb, Tq), the row
// maxima. Every thread computes the same result.
struct RowTotals {
    float Tb, Tq, W, C, P, carried;
};

template <int NW>
__device__ __forceinline__ RowTotals merge_waves(const WaveState* sm) {
    RowTotals t;
    t.Tb = -INFINITY;
    t.Tq = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        t.Tb = fmaxf(t.Tb, sm[w].Kb);
        t.Tq = fmaxf(t.Tq, sm[w].Kq);
    }
    t.W = 0.0f;
    t.C = 0.0f;
    t.P = 0.0f;
    t.carried = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        if (sm[w].Kb == -INFINITY) continue;  // wave saw no element
        float W = sm[w].W, C = sm[w].C, P = sm[w].P;
        if (sm[w].Kb != t.Tb || sm[w].Kq != t.Tq) {
            const Rescale f = rescale_factors(sm[w].Kb, sm[w].Kq, t.Tb, t.Tq);
            t.carried += fmaxf(f.fw, f.fcc) * sm[w].carried + fabsf(f.fcw) * W;
            apply_rescale(W, C, P, f);
        } else {
            t.carried += sm[w].carried;
        }
        t.W += W;
        t.C += C;
        t.P += P;
    }
    return t;
}

// Second evaluation of a row whose fast-path result is ill-conditioned (the
// three criteria in the kernel's epilogue), by all threads of the row's
// workgroup, starting from the fast path's float64 log-normalisers lb, lq:
// per token a = z - lse in float64, p = e^a_b, q = e^a_q, d = a_b - a_q and
// the non-negative Bregman term p h(d) = p (e^-d - 1 + d) (as q - p + p d for
// |d| >= 1, where the three parts do not cancel and e^-d alone could
// overflow), all summed in float64 with Sp = sum p and Sq = sum q. Then
// KL = sum p h(d) / Sp - (rho - 1 - ln rho), rho = Sq / Sp: the exact
// divergence of the normalised distributions (the fast path's normalisers
// need not be exact), a sum of non-negative terms less a second-order
// correction, so no cancellation; the log-normalisers become lse + ln Sp and
// lse + ln Sq, exact to the float64 sums. Every thread returns the same values.
template <class TB, class TQ, int NW>
__device__ void retake_row(const typename TB::elem* __restrict__ rb, const typename TQ::elem* __restrict__ rq,
                           int64_t vocab, int tid, double (*sm)[NW], double& kld, double& lb, double& lq) {
    // kSteps elements per thread per step, all loads issued before any
    // arithmetic (each load instruction covers NW * 64 consecutive elements)
    constexpr int kSteps = 16;
    constexpr int64_t kNT = NW * 64;
    double v[3] = {0.0, 0.0, 0.0};  // sum p h(d), Sp, Sq
    for (int64_t i0 = tid; i0 < vocab; i0 += kNT * kSteps) {
        float zb[kSteps], zq[kSteps];
#pragma unroll
        for (int j = 0; j < kSteps; ++j) {
            const int64_t i = i0 + j * kNT;
            zb[j] = i < vocab ? load_elem(rb, i) : 0.0f;
            zq[j] = i < vocab ? load_elem(rq, i) : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < kSteps; ++j) {
            if (i0 + j * kNT >= vocab) break;
            const double ab = static_cast<double>(zb[j]) - lb;
            const double aq = static_cast<double>(zq[j]) - lq;
            const double p = exp(ab), q = exp(aq), d = ab - aq;
            v[0] += fabs(d) < 1.0 ? p * (expm1(-d) + d) : (q - p) + p * d;
            v[1] += p;
            v[2] += q;
        }
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) {
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) v[k] += __shfl_xor(v[k], o);
    }
    if (NW > 1) {
        if ((tid & 63) == 0) {
#pragma unroll
            for (int k = 0; k < 3; ++k) sm[k][tid >> 6] = v[k];
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            v[k] = sm[k][0];
#pragma unroll
            for (int w = 1; w < NW; ++w) v[k] += sm[k][w];
        }
    }
    const double rho = v[2] / v[1];
    kld = v[0] / v[1] - (rho - 1.0 - log(rho));
    lb += log(v[1]);
    lq += log(v[2]);
}

template <class TB, class TQ, int NW, int U, int D, int MINW>
__global__ void __launch_bounds__(NW * 64, MINW)
    kld_rows_kernel(const typename TB::elem* __restrict__ base, const typename TQ::elem* __restrict__ quant,
                    int64_t vocab, int vec_ok, int64_t row_offset, RowOut out, unsigned int sel_lo_bits,
                    unsigned int sel_hi_bits) {
    constexpr bool kContig8 = std::is_same<TB, TBF16>::value && std::is_same<TQ, TBF16>::value;
    using LB = Tile<TB, kContig8>;
    using LQ = Tile<TQ, kContig8>;
    constexpr int NT = NW * 64;

    __shared__ WaveState sm_state[NW];
    __shared__ int sm_idx[NW][2];
    __shared__ double sm_retake[3][NW];
    __shared__ double sm_l2[NT * 3];  // per lane: second-level W2, C2, P2

    const int64_t r = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave index as a scalar: the wave's row pointers below are then scalar
    // too, and every load is a scalar base plus the lane's 32-bit offset
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const typename TB::elem* rb = base + r * vocab;
    const typename TQ::elem* rq = quant + r * vocab;

    LaneState st;
    st.Kb = -INFINITY;
    st.carried = 0.0f;
    st.Kq = -INFINITY;
    st.bestb = -INFINITY;
    st.bestq = -INFINITY;
    st.idxb = INT32_MAX;
    st.idxq = INT32_MAX;
#pragma unroll
    for (int s = 0; s < kSlots; ++s) {
        st.acc.W[s] = 0.0f;
        st.acc.C[s] = 0.0f;
        st.acc.P[s] = 0.0f;
    }
    st.l2 = &sm_l2[3 * tid];  // touched by this lane only
    st.l2[0] = 0.0;
    st.l2[1] = 0.0;
    st.l2[2] = 0.0;

    // ---- vector part: full wave-tiles, 16-byte loads ----
    const int64_t n_wt = vec_ok ? vocab / kWaveTile : 0;
    const int nt_w = (n_wt > wave) ? static_cast<int>((n_wt - wave + NW - 1) / NW) : 0;
    const int nfull = nt_w / U;
    const int64_t tile_stride = static_cast<int64_t>(NW) * kWaveTile;
    const typename TB::elem* wb = rb + static_cast<int64_t>(wave) * kWaveTile;
    const typename TQ::elem* wq = rq + static_cast<int64_t>(wave) * kWaveTile;

    // Selectors for the bf16-pair path, held in vector registers: a VOP3P
    // instruction may read only one scalar operand on this architecture, and
    // that slot is kept for the (wave-uniform) shift.
    unsigned int slo, shi;
    asm volatile("v_mov_b32 %0, %1" : "=v"(slo) : "s"(sel_lo_bits));
    asm volatile("v_mov_b32 %0, %1" : "=v"(shi) : "s"(sel_hi_bits));
    (void)slo;
    (void)shi;

    if (nfull > 0) {
        // D register sets used as a ring: while chunk c is processed the
        // loads of chunks c + 1 .. c + D - 1 are in flight. Chunk j lives in
        // set j % D; the steady loop is unrolled D times so that every set
        // index is a compile-time constant and every load in it is
        // unconditional (which keeps the compiler's vmcnt waits exact).
        typename LB::Raw ring_b[D][U];
        typename LQ::Raw ring_q[D][U];
        // Inside the loop a record is the code c * 8U + slot; it is turned
        // into an element index once the loop is done.
        auto chunk_index = [&](int c) {
            return [=](int i) -> int { return c * (U * 8) + i; };
        };
        auto load = [&](typename LB::Raw (&xb)[U], typename LQ::Raw (&xq)[U], int c) {
            const int64_t off = static_cast<int64_t>(c * U) * tile_stride;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                xb[u] = LB::load(wb + off + u * tile_stride, lane);
                xq[u] = LQ::load(wq + off + u * tile_stride, lane);
            }
        };
        auto process = [&](const typename LB::Raw (&xb)[U], const typename LQ::Raw (&xq)[U], int c) {
            if constexpr (kContig8) {
                u32x4 pb[U], pq[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    pb[u] = xb[u].v;
                    pq[u] = xq[u].v;
                }
                chunk_update_bf16_pairs<U>(pb, pq, st, chunk_index(c), slo, shi);
            } else {
                float zb[U * 8], zq[U * 8];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    LB::unpack(xb[u], &zb[u * 8]);
                    LQ::unpack(xq[u], &zq[u * 8]);
                }
                chunk_update<U * 8, false>(zb, zq, st, chunk_index(c));
            }
        };
#pragma unroll
        for (int k = 0; k < D - 1; ++k)
            if (k < nfull) load(ring_b[k], ring_q[k], k);
        // Issue priority. Waves of equal priority on a SIMD are issued oldest
        // first, so with the VALU busy the oldest wave streams fastest and a
        // launch's rows finish staggered: its last rows then run with few
        // waves per SIMD, each unable to keep enough loads in flight alone.
        // Lowering a wave's priority over the last quarter of its row lets
        // the waves that started later catch up, so the rows sharing a SIMD
        // finish closer together. (Priorities only order issue; the
        // arithmetic and its order are unchanged.)
        const int prio_2 = (3 * nfull / 4) / D * D, prio_1 = (7 * nfull / 8) / D * D,
                  prio_0 = (15 * nfull / 16) / D * D;
        __builtin_amdgcn_s_setprio(3);
        int c = 0;
        static_assert(kFoldChunks % D == 0, "folds fall on the steady loop's steps");
        for (; c + 2 * D - 2 < nfull; c += D) {
            if (c == prio_2) __builtin_amdgcn_s_setprio(2);
            if (c == prio_1) __builtin_amdgcn_s_setprio(1);
            if (c == prio_0) __builtin_amdgcn_s_setprio(0);
            if (c != 0 && c % kFoldChunks == 0) fold_slots(st.acc, st.l2);
#pragma unroll
            for (int k = 0; k < D; ++k) {
                load(ring_b[(k + D - 1) % D], ring_q[(k + D - 1) % D], c + k + D - 1);
                process(ring_b[k], ring_q[k], c + k);
            }
        }
        // fewer than 2D - 1 chunks remain; c is a multiple of D
#pragma unroll
        for (int t = 0; t < 2 * D - 2; ++t) {
            if (c + t < nfull) {
                if (c + t + D - 1 < nfull) load(ring_b[(t + D - 1) % D], ring_q[(t + D - 1) % D], c + t + D - 1);
                process(ring_b[t % D], ring_q[t % D], c + t);
            }
        }
    }
    {
        // element index of slot i % 8 of tile i / 8 of chunk c, for c * 8U + i
        auto decode = [&](int code) -> int {
            if (code == INT32_MAX) return code;
            const int c = code / (U * 8), i = code % (U * 8);
            const int64_t k = wave + static_cast<int64_t>(c * U + i / 8) * NW;
            return static_cast<int>(k * kWaveTile + tile_pos<kContig8>(lane, i % 8));
        };
        st.idxb = decode(st.idxb);
        st.idxq = decode(st.idxq);
    }
    for (int j = nfull * U; j < nt_w; ++j) {  // leftover single wave-tiles
        const int64_t off = static_cast<int64_t>(j) * tile_stride;
        typename LB::Raw xb = LB::load(wb + off, lane);
        typename LQ::Raw xq = LQ::load(wq + off, lane);
        float zb[8], zq[8];
        LB::unpack(xb, zb);
        LQ::unpack(xq, zq);
        const int64_t k = wave + static_cast<int64_t>(j) * NW;
        chunk_update<8, false>(zb, zq, st, [=](int i) -> int {
            return static_cast<int>(k * kWaveTile + tile_pos<kContig8>(lane, i));
        });
    }

    // ---- predicated part: elements [tail0, vocab) ----
    const int64_t tail0 = n_wt * kWaveTile;
    const int64_t rem = vocab - tail0;
    const int64_t n_tc = (rem + static_cast<int64_t>(NT) * kTailPerLane - 1) / (static_cast<int64_t>(NT) * kTailPerLane);
    // consecutive chunks alternate between the two halves of the slots, so
    // that a row taken entirely this way (unaligned pointers) spreads its
    // sums over all of them
    static_assert(2 * kTailPerLane == kSlots, "two chunks fill the slots");
    auto tail_chunk = [&](auto slot0, int64_t c) {
        float zb[kTailPerLane], zq[kTailPerLane];
#pragma unroll
        for (int s = 0; s < kTailPerLane; ++s) {
            const int64_t i = tail0 + (c * kTailPerLane + s) * NT + tid;
            const bool ok = i < vocab;
            zb[s] = ok ? load_elem(rb, i) : -INFINITY;
            zq[s] = ok ? load_elem(rq, i) : -INFINITY;
        }
        chunk_update<kTailPerLane, true, decltype(slot0)::value>(zb, zq, st, [=](int s) -> int {
            return static_cast<int>(tail0 + (c * kTailPerLane + s) * NT + tid);
        });
    };
    for (int64_t c = 0; c < n_tc; c += 2) {
        if (c != 0 && c % (2 * kFoldChunks) == 0) fold_slots(st.acc, st.l2);
        tail_chunk(std::integral_constant<int, 0>{}, c);
        if (c + 1 < n_tc) tail_chunk(std::integral_constant<int, kTailPerLane>{}, c + 1);
    }

    // ---- wave totals, then workgroup merge ----
    float W = 0.0f, C = 0.0f, P = 0.0f;
#pragma unroll
    for (int s = 0; s < kSlots; ++s) {
        W += st.acc.W[s];
        C += st.acc.C[s];
        P += st.acc.P[s];
    }
    W = static_cast<float>(static_cast<double>(W) + st.l2[0]);
    C = static_cast<float>(static_cast<double>(C) + st.l2[1]);
    P = static_cast<float>(static_cast<double>(P) + st.l2[2]);
    W = wave_sum(W);
    C = wave_sum(C);
    P = wave_sum(P);
    const float carried = wave_sum(st.carried);
    if (lane == 0) sm_state[wave] = WaveState{st.Kb, st.Kq, W, C, P, carried};
    __syncthreads();
    const RowTotals tot = merge_waves<NW>(sm_state);

    // ---- argmax: lowest index attaining the row maximum ----
    int candb = (st.bestb == tot.Tb) ? st.idxb : INT32_MAX;
    int candq = (st.bestq == tot.Tq) ? st.idxq : INT32_MAX;
    candb = wave_min_i(candb);
    candq = wave_min_i(candq);
    if (lane == 0) {
        sm_idx[wave][0] = candb;
        sm_idx[wave][1] = candq;
    }
    __syncthreads();

    // ---- per-row results: every thread computes the same values ----
    int ib = INT32_MAX, iq = INT32_MAX;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        ib = min(ib, sm_idx[w][0]);
        iq = min(iq, sm_idx[w][1]);
    }
    // KL = ln2 P/W - B, B = x - log1p(x), x = C/W; lse from the shifts and sums
    const double Wd = tot.W, Cd = tot.C, Pd = tot.P;
    const double x = Cd / Wd;
    const double B = x - log1p(x);
    double kld = 0.6931471805599453 * Pd / Wd - B;
    double lse_bd = static_cast<double>(tot.Tb) + log(Wd);
    double lse_qd = static_cast<double>(tot.Tq) + log(Wd + Cd);
    // Conditioning. The fp32 sums' relative error e (about one ulp, 1e-7, as
    // measured on the worst-conditioned rows found) reaches the result
    // amplified by amp = 2 (KL + B) + |x| (2 + x) / (1 + x): from P through
    // ln2 P / W = KL + B, from C through both log1p(x) and x. amp is large
    // only where the two rows' masses relative to their maxima differ
    // greatly (x far above 0: a much flatter quantized row; x near -1: a much
    // flatter base row). Rows with amp > 50 |KL| + 20 are taken again -- those
    // where the measured error, up to 1e-7 amp, could pass 5e-6 |KL| + 2e-6;
    // the rows that failed 1e-5 |KL| + 1e-7 had amp 800-6000, while the tails
    // of realistic rows (the two rows' top probabilities within a factor of 2)
    // stay below 5 -- and so are rows with 1 + x = (W + C) / W < 1/4, whose
    // quant normaliser log(W + C) has lost more than two bits to the
    // cancellation in W + C. Third, rescales move mass |fcw| W between W and C
    // (one row's maximum jumping while the other's stays): C keeps that mass's
    // rounding -- the product's and the sum's, ~1.2e-7 of it -- as absolute
    // error (later rescales scale it as they scale C and P; `carried`
    // follows), and P the rounding of the matching log2(e) (cw C + pw W)
    // terms, of the same size. Rows are taken again where that error could
    // exceed half the normaliser bound 2^-21 |lse| + 1e-6 of log(W + C) --
    // the mass was large and W + C ends small -- or the divergence's own
    // bound 1e-5 |KL| + 1e-7, which it reaches through P with weight 1 / W and
    // through C with |x| / (1 + x) / W (counted at half: the two share
    // roundings). The second catches a KL of ~0.1 over logits near 1e4, where
    // the normaliser bound is loose.
    const double amp = 2.0 * (fabs(kld) + B) + fabs(x) * (2.0 + x) / (1.0 + x);
    const double lse_tol = 4.76837158203125e-07 * fmax(fabs(lse_qd), 1.0) + 1e-6;
    const double moved = 1.2e-7 * static_cast<double>(tot.carried);
    const double opx = 1.0 + x;  // > 0: the second test below is multiplied through by it
    const unsigned int flags =
        (amp > 50.0 * fabs(kld) + 20.0 ? kRowFlagAmplified : 0u) | (opx < 0.25 ? kRowFlagQuantMass : 0u) |
        (moved > 0.5 * lse_tol * (Wd + Cd) || moved * (opx + 0.5 * fabs(x)) > (1e-5 * fabs(kld) + 1e-7) * Wd * opx
             ? kRowFlagCarried
             : 0u);
    if (__builtin_amdgcn_readfirstlane(flags) != 0u)  // the same in every wave of the workgroup
        retake_row<TB, TQ, NW>(rb, rq, vocab, tid, sm_retake, kld, lse_bd, lse_qd);

    if (tid == 0) {
        const float kl = static_cast<float>(kld);
        const uint8_t m = static_cast<uint8_t>(ib == iq);
        const int64_t g = row_offset + r;
        if (out.retake) out.retake[g] = static_cast<uint8_t>(flags);
        out.kld[g] = kl;
        out.match[g] = m;
        if (out.argmax_b) out.argmax_b[g] = ib;
        if (out.argmax_q) out.argmax_q[g] = iq;
        if (out.lse_b) out.lse_b[g] = lse_bd;
        if (out.lse_q) out.lse_q[g] = lse_qd;
        if (out.kld_out) out.kld_out[r] = kl;
        if (out.match_out) out.match_out[r] = m;
        if (out.argmax_b_out) out.argmax_b_out[r] = ib;
        if (out.argmax_q_out) out.argmax_q_out[r] = iq;

        // Token-conditioned values: log-probability of the actual next token
        // under each model and the change of its probability, from the two
        // gathered logits and the float64 log-normalisers.
        uint8_t ts = 0;
        float lpb = __builtin_nanf(""), lpq = __builtin_nanf(""), dpv = __builtin_nanf("");
        if (out.tokens) {
            const int32_t t = out.tokens[r];
            if (t >= vocab) {
                ts = 2;
            } else if (t >= 0) {
                ts = 1;
                const double a = static_cast<double>(load_elem(rb, t)) - lse_bd;
                const double b = static_cast<double>(load_elem(rq, t)) - lse_qd;
                lpb = static_cast<float>(a);
                lpq = static_cast<float>(b);
                dpv = static_cast<float>(exp(b) - exp(a));
            }
        }
        if (out.tok_state) {
            out.tok_state[g] = ts;
            out.logp_b[g] = lpb;
            out.logp_q[g] = lpq;
            out.dp[g] = dpv;
        }
        if (out.logp_b_out) out.logp_b_out[r] = lpb;
        if (out.logp_q_out) out.logp_q_out[r] = lpq;
        if (out.dp_out) out.dp_out[r] = dpv;
    }
}

template <class TB, class TQ, int NW, int U, int D, int MINW>
hipError_t launch_typed(const void* base, const void* quant, int64_t vocab, int64_t n_rows, int64_t row_offset,
                        const RowOut& out, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    const bool vec_ok = (vocab % 8 == 0) && (reinterpret_cast<uintptr_t>(base) % 16 == 0) &&
                        (reinterpret_cast<uintptr_t>(quant) % 16 == 0);
    if (start || stop)  // the dispatch records the events itself
        hipExtLaunchKernelGGL((kld_rows_kernel<TB, TQ, NW, U, D, MINW>), dim3(static_cast<unsigned>(n_rows)),
                              dim3(NW * 64), 0, stream, start, stop, 0,
                              static_cast<const typename TB::elem*>(base),
                              static_cast<const typename TQ::elem*>(quant), vocab, vec_ok ? 1 : 0, row_offset, out,
                              0x00003f80u /* bf16 pair (1, 0) */, 0x3f800000u /* bf16 pair (0, 1) */);
    else
        hipLaunchKernelGGL((kld_rows_kernel<TB, TQ, NW, U, D, MINW>), dim3(static_cast<unsigned>(n_rows)),
                           dim3(NW * 64), 0, stream, static_cast<const typename TB::elem*>(base),
                           static_cast<const typename TQ::elem*>(quant), vocab, vec_ok ? 1 : 0, row_offset, out,
                           0x00003f80u /* bf16 pair (1, 0) */, 0x3f800000u /* bf16 pair (0, 1) */);
    return hipGetLastError();
}

}  // namespace

// Launch shapes measured on MI355X (8192 x 151936 bf16 pairs; 16384 x 151936
// f32/bf16 pairs; 64 x 32000 f32 pairs): with both rows in bf16 one wave per
// row streams best once there are enough rows to give every SIMD several of
// them (fewer rows: split each row over more waves); rows with an f32 side
// carry 1.5-2x the bytes per element and run best with four waves per row
// and a two-deep ring (deeper rings cost them occupancy).
// The shape decides the summation order, so it is keyed on shape_rows (the
// handle's capacity), not on the rows of one call: any chunking of the same
// rows into one handle gives bit-identical results.
int64_t rows_max_per_launch() { return max_blocks_per_launch(4 * 64); }

hipError_t launch_rows(int base_type, int quant_type, const void* base, const void* quant, int64_t vocab,
                       int64_t n_rows, int64_t row_offset, int64_t shape_rows, const RowOut& out,
                       hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    if (n_rows > rows_max_per_launch()) return hipErrorInvalidValue;
    if (base_type == kBF16 && quant_type == kBF16) {
        if (shape_rows >= 4096)
            return launch_typed<TBF16, TBF16, 1, KLD_BB_UNROLL, KLD_DEPTH, KLD_BB_MIN_WAVES>(base, quant, vocab, n_rows, row_offset, out, stream, start, stop);
        if (shape_rows >= 2048)
            return launch_typed<TBF16, TBF16, 2, KLD_BB_UNROLL, KLD_DEPTH, KLD_BB_MIN_WAVES>(base, quant, vocab, n_rows, row_offset, out, stream, start, stop);
        return launch_typed<TBF16, TBF16, 4, KLD_BB_UNROLL, KLD_DEPTH, KLD_BB_MIN_WAVES>(base, quant, vocab, n_rows, row_offset, out, stream, start, stop);
    }
    if (base_type == kF32 && quant_type == kF32)
        return launch_typed<TF32, TF32, 4, 2, 2, 3>(base, quant, vocab, n_rows, row_offset, out, stream, start, stop);
    if (base_type == kF32 && quant_type == kBF16)
        return launch_typed<TF32, TBF16, 4, 2, 2, 3>(base, quant, vocab, n_rows, row_offset, out, stream, start, stop);
    return launch_typed<TBF16, TF32, 4, 2, 2, 3>(base, quant, vocab, n_rows, row_offset, out, stream, start, stop);
}

}  // namespace kldk
