// gdn_device.h -- device helpers shared by the gfx950 kernels of libgdn.
//
// Wave64 cross-lane sums through DPP, bfloat16 <-> float conversion, 16-byte
// vector types and the MFMA operand types used for the Gram matrices of the
// WY prologue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

// ---------------------------------------------------------------- bfloat16
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// float -> bfloat16 bits, round to nearest even; NaN stays NaN (quiet bit set).
// Both results are formed and one is selected, so no lane branches.
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    const uint32_t u = __float_as_uint(f);
    const uint32_t rne = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    const uint32_t nan = (u >> 16) | 0x0040u;
    return (uint16_t)(((u & 0x7fffffffu) > 0x7f800000u) ? nan : rne);
}

// load 4 consecutive elements (bf16 or f32) as floats; p is 8 / 16 byte aligned
template <bool BF16>
__device__ __forceinline__ float4 load4(const void* base, size_t idx)
{
    if constexpr (BF16) {
        const uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + idx);
        return make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
    } else {
        return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + idx);
    }
}

template <bool BF16>
__device__ __forceinline__ float load1(const void* base, size_t idx)
{
    if constexpr (BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
    else return reinterpret_cast<const float*>(base)[idx];
}

template <bool BF16>
__device__ __forceinline__ void store1(void* base, size_t idx, float v)
{
    if constexpr (BF16) reinterpret_cast<uint16_t*>(base)[idx] = f32_to_bf16(v);
    else reinterpret_cast<float*>(base)[idx] = v;
}

// ---------------------------------------------------------------- DPP sums
// DPP controls (GCN/CDNA encoding)
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <-> 7-i inside each group of 8
constexpr int kDppRowMirror = 0x140;     // lane i <-> 15-i inside each row of 16

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// sum over each aligned group of 8 lanes; every lane of the group gets it
__device__ __forceinline__ float sum8(float v)
{
    v += dpp_mov<kDppQuadXor1>(v);
    v += dpp_mov<kDppQuadXor2>(v);
    v += dpp_mov<kDppRowHalfMirror>(v);
    return v;
}

// sum over lanes l, l^16, l^32, l^48 (the four k-slices of an MFMA operand row)
__device__ __forceinline__ float sum_xor16_32(float v)
{
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}

// ---------------------------------------------------------------- misc
// 16-byte store; the non-temporal form streams past the caches
template <bool NT>
__device__ __forceinline__ void store_f4(float* p, f32x4_t v)
{
    if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(p));
    else *reinterpret_cast<f32x4_t*>(p) = v;
}

__device__ __forceinline__ f32x4_t load_f4(const float* p) { return *reinterpret_cast<const f32x4_t*>(p); }

}  // namespace gdn
