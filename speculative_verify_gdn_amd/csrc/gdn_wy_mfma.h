// gdn_wy_mfma.h -- helpers shared by the chunkwise (WY) prefill kernels:
// bf16 hi/lo splits of fp32 values, MFMA wrappers, the operand record order
// of q/k tiles in LDS, and the gates.
//
// Operand order.  A 32-wide slice of a contraction index is spread over the
// four lane groups g of a 16x16x32 MFMA operand as pi(g, s) = 4g + s (s < 4)
// and 16 + 4g + (s - 4) (s >= 4): the order in which two 16x16 accumulator
// tiles hold their rows, so accumulator tiles feed later products as operands
// directly.  fp32 operands enter the MFMA as a bf16 hi + lo pair; a product of
// two such pairs keeps the three largest partial products.
#pragma once

#include "gdn_device.h"

namespace gdn {
namespace wy {

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short bf16x4_t;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kBufferFlags = 0x00020000;  // buffer resource word 3: raw dword access on CDNA

__device__ __forceinline__ int pi_group(int x) { return (x & 15) >> 2; }
__device__ __forceinline__ int pi_slot(int x) { return ((x >> 4) << 2) | (x & 3); }

// record swizzle of q/k operand tiles (a permutation of the 64 records of slice m;
// it spreads the staging writes over the banks)
__device__ __forceinline__ int qk_rec(int lane, int m) { return lane ^ ((m & 3) << 2); }

// gates of one token: beta = sigmoid(raw beta), g = -softplus(alpha + dt_bias) e^{A_log}, with
// dtb = dt_bias and eal = e^{A_log} of the value head, read once per workgroup by the caller (a load
// in the chunk loop is repeated every chunk and waited for there); raw == false: the inputs are beta
// and g themselves
__device__ __forceinline__ void gate(float braw, float al, bool raw, float dtb, float eal, float& beta, float& g)
{
    if (raw) {
        beta = __frcp_rn(1.0f + __expf(-braw));
        const float a = al + dtb;
        const float sp = a > 20.0f ? a : __logf(1.0f + __expf(a));
        g = -sp * eal;
    } else {
        beta = braw;
        g = al;
    }
}

// dt_bias and e^{A_log} of value head h (zeros without raw gates)
__device__ __forceinline__ void head_gate_consts(const float* dt_bias, const float* A_log, int h, float& dtb,
                                                 float& eal)
{
    dtb = dt_bias != nullptr ? dt_bias[h] : 0.f;
    eal = dt_bias != nullptr ? __expf(A_log[h]) : 0.f;
}

// value head of workgroup row y: the value heads of key head kh sit at rows congruent mod 8
// (each block of 8 G rows holds 8 key heads, G = Hv / Hk), so with one workgroup per head and
// sequence they are dispatched to one XCD and read q, k from its L2; other shapes keep the identity
__device__ __forceinline__ int head_of_row(int y, int Hv, int Hk, int gx)
{
    const int G = Hv / Hk;
    if (gx != 1 || Hv % (8 * G) != 0) return y;
    const int k = y / (8 * G), r = y % (8 * G);
    return (8 * k + r % 8) * G + r / 8;
}

// bf16 hi (round to nearest) and lo (the rounded remainder) of 2 floats, packed
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo)
{
    const bf16x2_t hb = {(__bf16)x0, (__bf16)x1};
    uint32_t hu = __builtin_bit_cast(uint32_t, hb);
    // both packed words opaque: otherwise the compiler converts each value on its own (a convert with a
    // zero partner per value, then a byte permute to pack them), 8 instructions a pair instead of 6
    asm("" : "+v"(hu));
    const float r0 = x0 - __uint_as_float(hu << 16);
    const float r1 = x1 - __uint_as_float(hu & 0xffff0000u);
    const bf16x2_t lb = {(__bf16)r0, (__bf16)r1};
    uint32_t lu = __builtin_bit_cast(uint32_t, lb);
    asm("" : "+v"(lu));
    hi = hu;
    lo = lu;
}

__device__ __forceinline__ void split4(const f32x4_t x, uint2& hi, uint2& lo)
{
    split2(x[0], x[1], hi.x, lo.x);
    split2(x[2], x[3], hi.y, lo.y);
}

__device__ __forceinline__ bf16x4_t as4(uint2 u) { return __builtin_bit_cast(bf16x4_t, u); }

__device__ __forceinline__ bf16x8_t as8(uint2 a, uint2 b)
{
    return __builtin_bit_cast(bf16x8_t, make_uint4(a.x, a.y, b.x, b.y));
}

__device__ __forceinline__ f32x4_t mfma16(uint2 a, uint2 b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as4(a), as4(b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma32(bf16x8_t a, bf16x8_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float4 lds_f4(const float* p) { return *reinterpret_cast<const float4*>(p); }

// sum over each aligned group of N lanes (N = 4, 8 or 16), every lane gets it
template <int N>
__device__ __forceinline__ float group_sum(float v)
{
    v += dpp_mov<kDppQuadXor1>(v);
    v += dpp_mov<kDppQuadXor2>(v);
    if constexpr (N >= 8) v += dpp_mov<kDppRowHalfMirror>(v);
    if constexpr (N >= 16) v += dpp_mov<kDppRowMirror>(v);
    return v;
}

// acc + sum of squares of 8 bf16 (exact products, fp32 sums)
__device__ __forceinline__ float sq8(const uint4 u, float acc)
{
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const bf16x2_t v = __builtin_bit_cast(bf16x2_t, w[e]);
        acc = __builtin_amdgcn_fdot2_f32_bf16(v, v, acc, false);
    }
    return acc;
}

}  // namespace wy
}  // namespace gdn
