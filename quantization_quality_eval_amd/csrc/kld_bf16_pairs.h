// Packed bfloat16 pairs (two values per 32-bit word, the lower index in the
// low half): helpers shared by the kernels that stream bf16 rows.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

namespace kldk {
namespace pairs {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(unsigned int w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned int w) { return __uint_as_float(w & 0xffff0000u); }

// z - K for the eight values of r: v_dot2_f32_bf16(pair, (1, 0), -K) = lo - K
// and v_dot2_f32_bf16(pair, (0, 1), -K) = hi - K with the selectors slo, shi
// (bf16 pairs (1, 0) and (0, 1) held in vector registers). The products by 1
// and 0 are exact, so the result equals the fp32 subtraction whenever that is
// exact and differs from it by the direction of rounding otherwise; it is 0
// exactly at z == K and > 0 exactly when z > K.
//
// The three-operand VOP3P form is written out: left to itself the compiler
// turns the builtin into the two-address v_dot2c form and copies -K into
// every accumulator first, which costs what the fusion saves. One block forms
// the eight shifted values of a tile; it ends with s_nop 2 because a DOT
// result needs three wait states before another VALU instruction may read it,
// and the compiler does not see inside the block to add them. Pure ALU, no
// memory access; the shift is the single scalar operand.
__device__ __forceinline__ void shifted_tile(const u32x4& r, unsigned int slo, unsigned int shi, float negk,
                                             float* x) {
    asm("v_dot2_f32_bf16 %0, %8, %12, %14\n\t"
        "v_dot2_f32_bf16 %1, %8, %13, %14\n\t"
        "v_dot2_f32_bf16 %2, %9, %12, %14\n\t"
        "v_dot2_f32_bf16 %3, %9, %13, %14\n\t"
        "v_dot2_f32_bf16 %4, %10, %12, %14\n\t"
        "v_dot2_f32_bf16 %5, %10, %13, %14\n\t"
        "v_dot2_f32_bf16 %6, %11, %12, %14\n\t"
        "v_dot2_f32_bf16 %7, %11, %13, %14\n\t"
        "s_nop 2"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]),
          "=&v"(x[7])
        : "v"(r.x), "v"(r.y), "v"(r.z), "v"(r.w), "v"(slo), "v"(shi), "s"(negk));
}

// First slot (in index order) of a chunk of packed bf16 pairs holding m, from
// the bit patterns: m is a bf16 value, so z == m exactly when the 16-bit
// patterns agree, or when both are zeros of either sign.
template <int U>
__device__ __forceinline__ int first_pair_slot(const u32x4 (&r)[U], float m) {
    const unsigned int mb = __float_as_uint(m) >> 16;
    const unsigned int care = (mb & 0x7fffu) == 0 ? 0x7fffu : 0xffffu;  // +-0 match each other
    const unsigned int key = mb & care;
    unsigned int mask = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const unsigned int w[4] = {r[u].x, r[u].y, r[u].z, r[u].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            mask |= static_cast<unsigned int>((w[k] & care) == key) << (u * 8 + 2 * k);
            mask |= static_cast<unsigned int>(((w[k] >> 16) & care) == key) << (u * 8 + 2 * k + 1);
        }
    }
    return mask ? __builtin_ctz(mask) : U * 8;
}

// Largest value of a chunk of packed bf16 pairs.
template <int U>
__device__ __forceinline__ float exact_max(const u32x4 (&r)[U]) {
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        m = fmaxf(m, fmaxf(fmaxf(bf16_lo(r[u].x), bf16_hi(r[u].x)), fmaxf(bf16_lo(r[u].y), bf16_hi(r[u].y))));
        m = fmaxf(m, fmaxf(fmaxf(bf16_lo(r[u].z), bf16_hi(r[u].z)), fmaxf(bf16_lo(r[u].w), bf16_hi(r[u].w))));
    }
    return m;
}

}  // namespace pairs
}  // namespace kldk
