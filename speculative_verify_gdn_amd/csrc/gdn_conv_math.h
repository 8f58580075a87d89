// gdn_conv_math.h -- the float arithmetic of the conv step, shared by the
// conv kernels and the fused verify step so that both give the same bits.
//   pre  = fmaf chain over the taps, oldest first, starting from 0
//   silu = pre / (1 + e^-pre) with the exp below and IEEE division
// (every translation unit that includes this is compiled with
// -ffp-contract=off, IEEE fp32 division and fp32 denormals kept)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_device.h"

namespace gdn {

// e^x for the SiLU of the conv step.
// Cody-Waite reduction x = n ln2 + r with |r| <= ln2/2; degree-7 Taylor
// polynomial of e^r in Horner form with fused multiply-adds; exact scaling by
// 2^n split in two powers of two so that a subnormal result is rounded once.
//   kLog2e = nearest float to 1/ln 2
//   kLn2Hi = ln 2 rounded to a multiple of 2^-16 (n * kLn2Hi exact for |n| < 256)
//   kLn2Lo = nearest float to ln 2 - kLn2Hi
//   Taylor coefficients 1/k!, each the nearest float
__device__ __forceinline__ float conv_exp(float x)
{
    constexpr float kLog2e = 0x1.715476p+0f;
    constexpr float kLn2Hi = 0x1.62e4p-1f;
    constexpr float kLn2Lo = 0x1.7f7d1cp-20f;
    // the special ranges are selected at the end instead of branching; inside
    // (-104, 89) the clamp leaves x unchanged (a NaN clamps to -104 and is
    // replaced by itself below)
    const float xc = fminf(fmaxf(x, -104.0f), 89.0f);
    const float n = __builtin_rintf(xc * kLog2e);
    float r = __builtin_fmaf(-n, kLn2Hi, xc);
    r = __builtin_fmaf(-n, kLn2Lo, r);
    float p = 1.0f / 5040.0f;
    p = __builtin_fmaf(p, r, 1.0f / 720.0f);
    p = __builtin_fmaf(p, r, 1.0f / 120.0f);
    p = __builtin_fmaf(p, r, 1.0f / 24.0f);
    p = __builtin_fmaf(p, r, 1.0f / 6.0f);
    p = __builtin_fmaf(p, r, 1.0f / 2.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    const int ni = (int)n;
    const int n1 = ni / 2;
    const int n2 = ni - n1;
    const float s1 = __uint_as_float((uint32_t)(n1 + 127) << 23);
    const float s2 = __uint_as_float((uint32_t)(n2 + 127) << 23);
    float y = (p * s1) * s2;
    y = x >= 89.0f ? __builtin_inff() : y;
    y = x <= -104.0f ? 0.0f : y;
    return x != x ? x : y;
}

__device__ __forceinline__ float conv_silu(float pre)
{
    const float e = conv_exp(-pre);
    const float den = 1.0f + e;
    return pre / den;
}

// bf16(conv_silu(pre)), bit for bit, for bfloat16 outputs.  A fast estimate s
// from the hardware exp2 and reciprocal comes with a bound d on its distance to
// conv_silu(pre), so the exact value lies in [s - d, s + d].  Round to nearest
// even is odd-symmetric, so the magnitude is rounded and the sign put back.  On
// positive floats it is monotone in the bit pattern u: every value whose u has
// no tie point (low 16 bits 0x8000) between those of |s| - d and |s| + d rounds
// to (u + 0x8000) >> 16, the same for all of them.  (u + 0x7fff) >> 16 of the
// lower end equals that of the upper end exactly when there is no such tie (a
// tie at the lower end itself gives one less), so the fast result is taken
// only then; otherwise (or outside the range the bound covers, NaN and
// infinities included) the exact path decides.  The bound, relative to |s|,
// with x = -pre log2(e):
//   estimate:  x rounded (2^-23 |x| relative: the product and the constant),
//              so e^.. off by |x| ln2 2^-23; exp2 and rcp within 2 ulp each;
//              1 + e and pre * r rounded once each: < |x| 2^-23.5 + 2^-20.6
//   exact path: its exp within 1.5 ulp of e^x, two roundings: < 2^-21.4
// d = |s| (|x| 2^-22 + 2^-18) is more than twice their sum, and below |s|.
// For |pre| <= 64 every intermediate is a normal float.
__device__ __forceinline__ uint16_t conv_silu_bf16(float pre)
{
    const float ap = fabsf(pre);
    const float x = pre * -1.44269504f;
    const float e = __builtin_amdgcn_exp2f(x);
    const float s = pre * __builtin_amdgcn_rcpf(1.0f + e);
    const float as = fabsf(s);
    const float d = as * __builtin_fmaf(fabsf(x), 0x1p-22f, 0x1p-18f);
    const uint32_t lo = (__float_as_uint(as - d) + 0x7fffu) >> 16;
    const uint32_t hi = (__float_as_uint(as + d) + 0x8000u) >> 16;
    const bool fast = (ap <= 64.0f) & (ap >= 0x1p-60f) & (lo == hi);
    uint16_t out = (uint16_t)(hi | ((__float_as_uint(s) >> 16) & 0x8000u));
    if (__builtin_expect(!fast, 0)) out = f32_to_bf16(conv_silu(pre));
    return out;
}

// pre-activation of one channel over a window of W rows (oldest first)
template <int W>
__device__ __forceinline__ float conv_pre(const float (&tap)[W], const float (&col)[W])
{
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < W; ++j) acc = __builtin_fmaf(tap[j], col[j], acc);
    return acc;
}

}  // namespace gdn
