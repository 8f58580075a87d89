// gdn_timeline.h -- optional wall-clock marks inside the fused verify step.
//
// Built only into the instrumented library (python -m speculative_verify_gdn_amd.build
// --timeline, which defines GDN_TIMELINE and links libgdn_timeline.so); the product
// library compiles every mark to nothing.  Each wave takes the 100 MHz real-time
// counter at mark n and, at its end (GDN_TL_END, after GDN_TL_BEGIN at its start),
// writes its marks into a device array indexed by (workgroup, wave, n), which
// gdn_timeline_read copies to the host.  Only workgroups below kTlGroups and
// waves below kTlWaves record.  GDN_TLV(n, v) places the mark after value v has arrived.
#pragma once

#include <hip/hip_runtime.h>

#ifdef GDN_TIMELINE
namespace gdn {
constexpr int kTlGroups = 2048, kTlWaves = 16, kTlMarks = 16;
// one array per translation unit (each has its own reader, GDN_TIMELINE_READER)
static __device__ unsigned long long g_timeline[kTlGroups * kTlWaves * kTlMarks];
}  // namespace gdn
// the host readers of this translation unit's marks: NAME_read(dst, bytes), NAME_clear()
#define GDN_TIMELINE_READER(NAME)                                                                        \
    extern "C" int NAME##_read(void* dst, size_t bytes)                                               \
    {                                                                                                  \
        if (bytes > sizeof(gdn::g_timeline)) bytes = sizeof(gdn::g_timeline);                          \
        return (int)hipMemcpyFromSymbol(dst, HIP_SYMBOL(gdn::g_timeline), bytes, 0, hipMemcpyDeviceToHost); \
    }                                                                                                  \
    extern "C" int NAME##_clear(void)                                                                 \
    {                                                                                                  \
        void* p = nullptr;                                                                             \
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(gdn::g_timeline));                           \
        if (e == hipSuccess) e = hipMemset(p, 0, sizeof(gdn::g_timeline));                             \
        return (int)e;                                                                                 \
    }
// the marks of a wave are held in lanes 0..kTlMarks-1 of two registers (counter high and low
// words) and written out once, at the wave's end: a store per mark would count in the wave's
// memory counter, and every later wait for a load would then also wait for those stores
#define GDN_TL_BEGIN()                                                                                 \
    unsigned gdn_tl_lo_ = 0, gdn_tl_hi_ = 0;                                                           \
    const unsigned gdn_tl_lane_ = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u))
#define GDN_TL(n)                                                                                      \
    do {                                                                                               \
        const unsigned long long t_ = __builtin_amdgcn_s_memrealtime();                                \
        gdn_tl_lo_ = gdn_tl_lane_ == (unsigned)(n) ? (unsigned)t_ : gdn_tl_lo_;                        \
        gdn_tl_hi_ = gdn_tl_lane_ == (unsigned)(n) ? (unsigned)(t_ >> 32) : gdn_tl_hi_;                \
    } while (0)
#define GDN_TL_END()                                                                                   \
    do {                                                                                               \
        const unsigned wg_ = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);          \
        const unsigned l_ = threadIdx.x & 63, w_ = threadIdx.x >> 6;                                   \
        if (l_ < (unsigned)gdn::kTlMarks && wg_ < (unsigned)gdn::kTlGroups && w_ < (unsigned)gdn::kTlWaves) \
            gdn::g_timeline[(wg_ * gdn::kTlWaves + w_) * gdn::kTlMarks + l_] =                          \
                ((unsigned long long)gdn_tl_hi_ << 32) | gdn_tl_lo_;                                   \
    } while (0)
// the mark once value v is available (an empty asm statement that takes v: the wait for the load
// that produces v is placed before the mark)
#define GDN_TLV(n, v)                              \
    do {                                           \
        asm volatile("" ::"v"(v));                 \
        GDN_TL(n);                                 \
    } while (0)
#else
#define GDN_TL_BEGIN() ((void)0)
#define GDN_TL_END() ((void)0)
#define GDN_TL(n) ((void)0)
#define GDN_TLV(n, v) ((void)0)
#endif
