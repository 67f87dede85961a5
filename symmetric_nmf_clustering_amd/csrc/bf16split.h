// Exact three-part bf16 split of fp32 values and the bf16 matrix-core step
// that consumes the parts (gfx950).
//
// An fp32 value x splits exactly into three bf16 parts, x = x1 + x2 + x3:
// x1 = bf16(x) rounded to nearest even, x2 = bf16(x - x1), x3 = bf16(x - x1 -
// x2). Each difference is exact in fp32, and x's 24-bit significand fits in
// the three 8-bit ones, so nothing is lost (for |x| above ~1e-31, where x3
// stays a normal bf16). With |x2| <= 2^-8 |x| and |x3| <= 2^-16 |x|, the
// product x y keeps the six terms x1y1, x1y2, x2y1, x1y3, x2y2, x3y1; the
// three it drops sum to at most ~2^-23 |x y|, about one fp32 rounding of the
// product. Each term is one v_mfma_f32_16x16x32_bf16 accumulating in fp32.
#pragma once

#include "common.h"

namespace symnmf {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// (a, b) -> the packed bf16 pairs of their three-part splits (element 0 of a
// pair in the low half, as the matrix core reads it).
__device__ __forceinline__ void split3_pair(float a, float b, uint32_t& p1, uint32_t& p2,
                                            uint32_t& p3) {
    const f32x2 v = {a, b};
    const bf16x2 h1 = __builtin_convertvector(v, bf16x2);  // round to nearest even
    const f32x2 r1 = v - __builtin_convertvector(h1, f32x2);  // exact
    const bf16x2 h2 = __builtin_convertvector(r1, bf16x2);
    const f32x2 r2 = r1 - __builtin_convertvector(h2, f32x2);  // exact
    const bf16x2 h3 = __builtin_convertvector(r2, bf16x2);     // exact
    p1 = __builtin_bit_cast(uint32_t, h1);
    p2 = __builtin_bit_cast(uint32_t, h2);
    p3 = __builtin_bit_cast(uint32_t, h3);
}

__device__ __forceinline__ void split3_8(const float (&v)[8], u32x4& x1, u32x4& x2, u32x4& x3) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t a, b, c;
        split3_pair(v[2 * q], v[2 * q + 1], a, b, c);
        x1[q] = a;
        x2[q] = b;
        x3[q] = c;
    }
}

__device__ __forceinline__ floatx4 mfma_bf16(const u32x4& a, const u32x4& b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// acc += x y over one 32-deep K block, x and y given by their three parts;
// the smallest terms first.
__device__ __forceinline__ floatx4 mfma_split6(const u32x4& a1, const u32x4& a2, const u32x4& a3,
                                               const u32x4& b1, const u32x4& b2, const u32x4& b3,
                                               floatx4 acc) {
    acc = mfma_bf16(a3, b1, acc);
    acc = mfma_bf16(a2, b2, acc);
    acc = mfma_bf16(a1, b3, acc);
    acc = mfma_bf16(a2, b1, acc);
    acc = mfma_bf16(a1, b2, acc);
    acc = mfma_bf16(a1, b1, acc);
    return acc;
}

}  // namespace symnmf
