// gdn_conv_math.h -- the float arithmetic of the conv step, shared by the
// conv kernels and the fused verify step so that both give the same bits.
//   pre  = fmaf chain over the taps, oldest first, starting from 0
//   silu = pre / (1 + e^-pre) with the exp below and IEEE division
// (every translation unit that includes this is compiled with
// -ffp-contract=off, IEEE fp32 division and fp32 denormals kept)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
