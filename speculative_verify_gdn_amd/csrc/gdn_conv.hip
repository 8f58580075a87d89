// gdn_conv.hip -- fused causal depthwise conv1d decode / verify step (gfx950).
//
// One kernel does what the pages describe as replacing transpose / concat /
// ssm_conv / silu / cpy: build the window [history ; new tokens], apply the
// W-tap depthwise conv and SiLU, write the history back in place and keep the
// whole window so that a partial accept can restore the conv state
// (lucebox PR #637, commit message on ggml_ssm_conv_step and the review note
// on its sources; atlas PR #297, commit message on
// causal_conv1d_update_prefill_inter).
//
// The result is bit-exact by construction: every rounding is fixed.
//   pre  = fmaf chain over the taps, oldest first, starting from 0
//   silu = pre / (1 + e^-pre) with the exp below and IEEE division
//   out  = round-to-nearest-even bfloat16 (or the float itself)
// This file is compiled with -ffp-contract=off, IEEE fp32 division and fp32
// denormals kept.
//
// Thread mapping: a thread owns 8 consecutive channels of one sequence and a
// segment of kSeg consecutive tokens; consecutive threads own consecutive
// channels, so every row access is one coalesced 16-byte (bf16) or 32-byte
// (f32) access per thread.  Segments after the first start at token
// kSeg >= W-1 and therefore never read the history; the first segment reads
// the old history and is also the only writer of the new one, so the in-place
// update has no race.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

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
    if (x != x) return x;
    if (x >= 89.0f) return __builtin_inff();
    if (x <= -104.0f) return 0.0f;
    const float n = __builtin_rintf(x * kLog2e);
    float r = __builtin_fmaf(-n, kLn2Hi, x);
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
    return (p * s1) * s2;
}

__device__ __forceinline__ float conv_silu(float pre)
{
    const float e = conv_exp(-pre);
    const float den = 1.0f + e;
    return pre / den;
}

constexpr int kCh = 8;    // channels per thread
constexpr int kSeg = 8;   // tokens per thread; must be >= W-1
constexpr int kThreads = 256;

template <bool BF16>
__device__ __forceinline__ void load_row8(const void* base, size_t off, int nch, bool vec, float v[kCh])
{
    if (vec) {
        if constexpr (BF16) {
            const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + off);
            v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x); v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
            v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z); v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
        } else {
            const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + off);
            const float4 b = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + off + 4);
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
            v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < kCh; ++e) v[e] = e < nch ? load1<BF16>(base, off + e) : 0.0f;
    }
}

template <bool BF16>
__device__ __forceinline__ void store_row8(void* base, size_t off, int nch, bool vec, const float v[kCh])
{
    if (vec) {
        if constexpr (BF16) {
            uint4 u;
            u.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
            u.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
            u.z = (uint32_t)f32_to_bf16(v[4]) | ((uint32_t)f32_to_bf16(v[5]) << 16);
            u.w = (uint32_t)f32_to_bf16(v[6]) | ((uint32_t)f32_to_bf16(v[7]) << 16);
            *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(base) + off) = u;
        } else {
            float* p = reinterpret_cast<float*>(base) + off;
            *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
            *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
        }
    } else {
#pragma unroll
        for (int e = 0; e < kCh; ++e)
            if (e < nch) store1<BF16>(base, off + e, v[e]);
    }
}

template <bool BF16, int W>
__global__ __launch_bounds__(kThreads) void conv_step_kernel(ConvArgs a)
{
    constexpr int R = kSeg + W - 1;  // window rows a thread touches
    const int c0 = (blockIdx.x * kThreads + threadIdx.x) * kCh;
    if (c0 >= a.C) return;
    const int b = blockIdx.z;
    const int t0 = blockIdx.y * kSeg;
    const int T = a.T, C = a.C;
    const int tn = min(kSeg, T - t0);
    const int nch = min(kCh, C - c0);
    const bool vec = (nch == kCh) && ((C & 7) == 0);
    const size_t xb = (size_t)b * T * C;
    const size_t hb = (size_t)b * (W - 1) * C;

    // window row r (absolute) is history row r for r < W-1, else token r-(W-1)
    float col[R][kCh];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int row = t0 + r;
        if (r < tn + W - 1) {
            if (row < W - 1) load_row8<BF16>(a.hist, hb + (size_t)row * C + c0, nch, vec, col[r]);
            else load_row8<BF16>(a.x, xb + (size_t)(row - (W - 1)) * C + c0, nch, vec, col[r]);
        }
    }
    float wt[kCh][W];
#pragma unroll
    for (int e = 0; e < kCh; ++e)
#pragma unroll
        for (int j = 0; j < W; ++j) wt[e][j] = e < nch ? a.w[(size_t)(c0 + e) * W + j] : 0.0f;

#pragma unroll
    for (int t = 0; t < kSeg; ++t) {
        if (t < tn) {
            float out[kCh];
#pragma unroll
            for (int e = 0; e < kCh; ++e) {
                float acc = 0.0f;
#pragma unroll
                for (int j = 0; j < W; ++j) acc = __builtin_fmaf(wt[e][j], col[t + j][e], acc);
                out[e] = conv_silu(acc);
            }
            store_row8<BF16>(a.y, xb + (size_t)(t0 + t) * C + c0, nch, vec, out);
        }
    }

    if (a.win) {
        const size_t wb = (size_t)b * (W - 1 + T) * C;
        // this thread's window rows t0 + W-1 .. t0 + W-1 + tn - 1 (its tokens)
#pragma unroll
        for (int t = 0; t < kSeg; ++t)
            if (t < tn) store_row8<BF16>(a.win, wb + (size_t)(t0 + W - 1 + t) * C + c0, nch, vec, col[t + W - 1]);
        if (t0 == 0) {
#pragma unroll
            for (int r = 0; r < W - 1; ++r) store_row8<BF16>(a.win, wb + (size_t)r * C + c0, nch, vec, col[r]);
        }
    }

    if (t0 == 0) {
        // new history = window rows T .. T+W-2; the old history is already in
        // registers, so overwriting it in place is safe
#pragma unroll
        for (int j = 0; j < W - 1; ++j) {
            const int row = T + j;
            float v[kCh];
            if (row < tn + W - 1) {
#pragma unroll
                for (int e = 0; e < kCh; ++e) v[e] = col[0][e];
#pragma unroll
                for (int r = 1; r < R; ++r)
                    if (r == row)
#pragma unroll
                        for (int e = 0; e < kCh; ++e) v[e] = col[r][e];
            } else {
                load_row8<BF16>(a.x, xb + (size_t)(row - (W - 1)) * C + c0, nch, vec, v);
            }
            store_row8<BF16>(a.hist, hb + (size_t)j * C + c0, nch, vec, v);
        }
    }
}

template <bool BF16>
hipError_t launch_w(const ConvArgs& a, hipStream_t s)
{
    const int groups = (a.C + kCh - 1) / kCh;
    dim3 grid((groups + kThreads - 1) / kThreads, (a.T + kSeg - 1) / kSeg, a.B);
    dim3 block(kThreads);
    switch (a.W) {
    case 2: conv_step_kernel<BF16, 2><<<grid, block, 0, s>>>(a); break;
    case 3: conv_step_kernel<BF16, 3><<<grid, block, 0, s>>>(a); break;
    case 4: conv_step_kernel<BF16, 4><<<grid, block, 0, s>>>(a); break;
    case 5: conv_step_kernel<BF16, 5><<<grid, block, 0, s>>>(a); break;
    case 6: conv_step_kernel<BF16, 6><<<grid, block, 0, s>>>(a); break;
    case 7: conv_step_kernel<BF16, 7><<<grid, block, 0, s>>>(a); break;
    case 8: conv_step_kernel<BF16, 8><<<grid, block, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_conv_step(const ConvArgs& a, bool bf16, hipStream_t s)
{
    return bf16 ? launch_w<true>(a, s) : launch_w<false>(a, s);
}

}  // namespace gdn
