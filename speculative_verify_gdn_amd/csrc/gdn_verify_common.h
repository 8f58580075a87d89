// gdn_verify_common.h -- device pieces shared by the chain verify kernels
// (gdn_verify.hip: the verify, tree and replay modes; gdn_step.hip: the fused
// verify step).  Both evaluate the same recurrence with the same reductions, so
// the fused step gives the bits of the separate calls.
#pragma once

#include "gdn_device.h"

namespace gdn {

constexpr int kWaves = 4;                // waves of one value head's row group
constexpr int kThreads = kWaves * 64;

// sum over each aligned group of N lanes (N = 4, 8, 16 or 32), every lane gets it
template <int N>
__device__ __forceinline__ float group_sum(float v)
{
    v += dpp_mov<kDppQuadXor1>(v);
    v += dpp_mov<kDppQuadXor2>(v);
    if constexpr (N >= 8) v += dpp_mov<kDppRowHalfMirror>(v);
    if constexpr (N >= 16) v += dpp_mov<kDppRowMirror>(v);
    if constexpr (N >= 32) {
        // the two rows of 16 lanes exchanged in one VALU instruction (each row now holds its sum in
        // every lane): the first result holds row 2m in both rows, the second row 2m+1, so their sum
        // is row 2m + row 2m+1 in every lane, the same bits as v + partner in either row
        const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(x[0]) + __uint_as_float(x[1]);
    }
    static_assert(N <= 32, "groups of at most 32 lanes");
    return v;
}

// inclusive prefix sum over lanes 0..N-1 (N = 16, 32 or 64; lanes past N get garbage):
// Hillis-Steele inside each DPP row of 16 lanes, then the totals of the earlier rows
// (their last lanes) added to each later row
template <int N>
__device__ __forceinline__ float lane_scan(float v)
{
    static_assert(N == 16 || N == 32 || N == 64, "one, two or four DPP rows");
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xF, 0xF, true));  // row_shr:1
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xF, 0xF, true));  // row_shr:2
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xF, 0xF, true));  // row_shr:4
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xF, 0xF, true));  // row_shr:8
    if constexpr (N >= 32) {
        const int row = __lane_id() >> 4;
        const float t0 = __shfl(v, 15, 64);
        if constexpr (N == 32) {
            v = row == 1 ? v + t0 : v;
        } else {
            const float t1 = __shfl(v, 31, 64), t2 = __shfl(v, 47, 64);
            const float carry = row == 0 ? 0.f : (row == 1 ? t0 : (row == 2 ? t0 + t1 : (t0 + t1) + t2));
            v += carry;
        }
    }
    return v;
}

// sum of squares of the 16 bytes of a q/k row piece (exact products, fp32 sums)
template <bool BF16>
__device__ __forceinline__ float sumsq16(const uint4 u)
{
    float s = 0.f;
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if constexpr (BF16) {
            typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
            const bf16x2_t v = __builtin_bit_cast(bf16x2_t, w[e]);
            s = __builtin_amdgcn_fdot2_f32_bf16(v, v, s, false);
        } else {
            const float f = __uint_as_float(w[e]);
            s = __builtin_fmaf(f, f, s);
        }
    }
    return s;
}

// gates of one token: raw (dtb, alog = the head's dt_bias and A_log) or, with
// raw false, beta and g given directly.  Both forms are formed and one selected:
// with no branch, nothing lets the compiler sink the loads of dtb and alog behind
// the gate data.
__device__ __forceinline__ void gate(float braw, float al, bool raw, float dtb, float alog, float& beta, float& g)
{
    const float br = __frcp_rn(1.0f + __expf(-braw));
    const float a = al + dtb;
    const float sp = a > 20.0f ? a : __logf(1.0f + __expf(a));
    const float gr = -sp * __expf(alog);
    beta = raw ? br : braw;
    g = raw ? gr : al;
}


// the raw bits of one element (bf16 zero-extended, or f32): loaded without a
// conversion, so that a load inside a branch is not waited for at its end
template <bool BF16>
__device__ __forceinline__ uint32_t ldraw(const void* base, size_t idx)
{
    if constexpr (BF16) return reinterpret_cast<const uint16_t*>(base)[idx];
    else return reinterpret_cast<const uint32_t*>(base)[idx];
}

template <bool BF16>
__device__ __forceinline__ float rawf(uint32_t u) { return __uint_as_float(BF16 ? u << 16 : u); }

template <bool BF16>
__device__ __forceinline__ void straw(void* base, size_t idx, uint32_t u)
{
    if constexpr (BF16) reinterpret_cast<uint16_t*>(base)[idx] = (uint16_t)u;
    else reinterpret_cast<uint32_t*>(base)[idx] = u;
}

template <bool IN_BF16>
__device__ __forceinline__ float4 lds4(const void* p)
{
    if constexpr (IN_BF16) {
        const uint2 u = *reinterpret_cast<const uint2*>(p);
        return make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
    } else {
        return *reinterpret_cast<const float4*>(p);
    }
}

}  // namespace gdn
