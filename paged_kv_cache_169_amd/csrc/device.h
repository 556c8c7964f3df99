// device.h -- small device helpers used by several kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace kvc {

// bf16 <-> fp32. bf16 is the upper half of an fp32, so widening is a shift.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// fp32 <-> IEEE binary16 bits. The hardware conversion rounds to nearest even
// (default MODE) and keeps fp16 subnormals.
__device__ __forceinline__ uint16_t f_to_f16_bits(float f) {
    _Float16 h = (_Float16)f;
    return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_bits_to_f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o));
    return v;
}
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

// KVQuant INT4 scale and min of a group whose min/max are known: s = (max -
// min) / 15 in fp32 (correctly rounded), both stored as fp16; a zero min or
// max of either sign is taken as +0, so the result does not depend on which
// zero a reduction returned.
struct Q4Params {
    uint16_t s16, m16;
    float s, m;  // the stored values, widened
    float r;     // hardware reciprocal of s (1 ulp), for q4_code's fast quotient
};
__device__ __forceinline__ Q4Params q4_params(float mn, float mx) {
    if (mn == 0.0f) mn = 0.0f;
    if (mx == 0.0f) mx = 0.0f;
    float s32 = __fdiv_rn(__fsub_rn(mx, mn), 15.0f);
    Q4Params p;
    p.s16 = f_to_f16_bits(s32);
    p.m16 = f_to_f16_bits(mn);
    p.s = f16_bits_to_f(p.s16);
    p.m = f16_bits_to_f(p.m16);
    p.r = p.s != 0.0f ? __builtin_amdgcn_rcpf(p.s) : 0.0f;
    return p;
}

// code = clamp(round((x - m) / s), 0, 15), rounding half away from zero, from
// the stored (fp16) m and s; every code is 0 when s is 0.
// The quotient is first taken through the hardware reciprocal: with a 1-ulp
// reciprocal, d * r lies within 2^-19 of the exact (x - m) / s for quotients
// below 16, and f1 = d * r + 0.5 (one fused multiply-add, one rounding at
// most 2^-20) within 2^-17 of the exact value plus one half. When f1's fraction is more
// than 2^-16 from an integer, floor(f1) is therefore the code itself; the
// few quotients that close to a half-integer take the correctly rounded
// division and the exact half-away rounding.
//
// q4_code_fast: floor(f1) before the clamp. worst keeps the largest
// |fraction(f1) - 1/2| seen; a value is near (one of those few) when that
// distance reaches 1/2 - 2^-16 (q4_near). (s = 0: r = 0 makes every
// quotient 0, f1 = 0.5, distance 0; a non-finite x gives NaN, which fmaxf
// ignores, and the clamp turns its code into 0.)
constexpr float kQ4NearTie = 0.5f - 0x1p-16f;
__device__ __forceinline__ float q4_code_fast(float x, const Q4Params &p, float &worst) {
    const float d = __fsub_rn(x, p.m);
    const float f1 = __fmaf_rn(d, p.r, 0.5f);
    const float c = floorf(f1);
    const float e = __fsub_rn(__fsub_rn(f1, c), 0.5f);  // both exact
    worst = fmaxf(worst, fabsf(e));
    return c;
}
__device__ __forceinline__ bool q4_near(float worst) { return worst >= kQ4NearTie; }
// The exact rounding, for the values q4_code_fast marks near.
__device__ __forceinline__ float q4_code_exact(float x, const Q4Params &p) {
    const float v = __fdiv_rn(__fsub_rn(x, p.m), p.s);
    const float t = truncf(v);  // v - t is exact
    return t + (__fsub_rn(v, t) >= 0.5f ? 1.0f : 0.0f);
}
__device__ __forceinline__ uint32_t q4_clamp(float c) {
    return (uint32_t)fminf(fmaxf(c, 0.0f), 15.0f);  // a NaN quotient gives 0
}
__device__ __forceinline__ uint32_t q4_code(float x, const Q4Params &p) {
    float worst = 0.0f;
    float c = q4_code_fast(x, p, worst);
    if (q4_near(worst)) c = q4_code_exact(x, p);
    return q4_clamp(c);
}

// The codes of N bf16 pairs w[i] (the low value coded with pa, the high one
// with pb) as bytes code[i] = low code | high code << 4. The same codes as
// q4_code, with the near-tie test of all 2N values behind one branch
// instead of one branch per value.
template <int N>
__device__ __forceinline__ void q4_code_pairs(const uint32_t (&w)[N], const Q4Params &pa, const Q4Params &pb,
                                              uint32_t (&code)[N]) {
    // codes are packed as soon as they are formed (few live registers)
    float worst = 0.0f;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float lo = q4_code_fast(bf16_lo(w[i]), pa, worst);
        const float hi = q4_code_fast(bf16_hi(w[i]), pb, worst);
        // the clamp as one median-of-three (a NaN operand gives the minimum
        // of the other two, 0, like q4_clamp), then both nibbles at once:
        // lo + 16 hi is an exact integer in [0, 255]
        const float cl = __builtin_amdgcn_fmed3f(lo, 0.0f, 15.0f), ch = __builtin_amdgcn_fmed3f(hi, 0.0f, 15.0f);
        code[i] = (uint32_t)__fmaf_rn(ch, 16.0f, cl);
    }
    if (q4_near(worst)) {  // rare: only the values near a tie take the exact division
#pragma unroll
        for (int i = 0; i < N; ++i) {
            float w0 = 0.0f, w1 = 0.0f;
            q4_code_fast(bf16_lo(w[i]), pa, w0);
            q4_code_fast(bf16_hi(w[i]), pb, w1);
            if (q4_near(w0)) code[i] = (code[i] & 0xf0u) | q4_clamp(q4_code_exact(bf16_lo(w[i]), pa));
            if (q4_near(w1)) code[i] = (code[i] & 0x0fu) | (q4_clamp(q4_code_exact(bf16_hi(w[i]), pb)) << 4);
        }
    }
}

// Lane mapping of the two coders below (one wave64 per row or block): lane l
// owns channel pair (2l, 2l+1), i.e. one 32-bit word of a bf16 row and one
// byte of a code row; for head_dim 64 lanes 32..63 idle (act false).

// Code one bf16 token row (one word per lane) per token into code row `dst`
// (one byte per lane) and the fp16 scale/min at *s16, *m16.
__device__ __forceinline__ void code_v_row(uint32_t w, bool act, uint8_t *dst, uint16_t *s16, uint16_t *m16,
                                           int lane) {
    const float x0 = bf16_lo(w), x1 = bf16_hi(w);
    float mn = act ? fminf(x0, x1) : INFINITY;
    float mx = act ? fmaxf(x0, x1) : -INFINITY;
    mn = wave_min(mn);
    mx = wave_max(mx);
    const Q4Params q = q4_params(mn, mx);
    if (act) dst[lane] = (uint8_t)(q4_code(x0, q) | (q4_code(x1, q) << 4));
    if (lane == 0) {
        *s16 = q.s16;
        *m16 = q.m16;
    }
}

// Code the K of one full block per channel. w[t] is this lane's word of token
// row t. Writes the 16 code rows (one byte per lane each) and the per-channel
// fp16 scale/min of channels 2*lane, 2*lane+1.
__device__ __forceinline__ void code_k_block(const uint32_t (&w)[kBlock], bool act, uint8_t *kq_tile,
                                             uint16_t *ks_row, uint16_t *km_row, int lane, int half_dim) {
    float mn0 = INFINITY, mx0 = -INFINITY, mn1 = INFINITY, mx1 = -INFINITY;
#pragma unroll
    for (int t = 0; t < kBlock; ++t) {
        const float a = bf16_lo(w[t]), b = bf16_hi(w[t]);
        mn0 = fminf(mn0, a);
        mx0 = fmaxf(mx0, a);
        mn1 = fminf(mn1, b);
        mx1 = fmaxf(mx1, b);
    }
    const Q4Params q0 = q4_params(mn0, mx0), q1 = q4_params(mn1, mx1);
    if (!act) return;
#pragma unroll
    for (int t = 0; t < kBlock; ++t)
        kq_tile[t * half_dim + lane] = (uint8_t)(q4_code(bf16_lo(w[t]), q0) | (q4_code(bf16_hi(w[t]), q1) << 4));
    reinterpret_cast<uint32_t *>(ks_row)[lane] = (uint32_t)q0.s16 | ((uint32_t)q1.s16 << 16);
    reinterpret_cast<uint32_t *>(km_row)[lane] = (uint32_t)q0.m16 | ((uint32_t)q1.m16 << 16);
}

}  // namespace kvc
