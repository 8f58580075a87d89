// gdn_timeline.h -- optional wall-clock marks inside the fused verify step.
//
// Built only into the instrumented library (python -m speculative_verify_gdn_amd.build
// --timeline, which defines GDN_TIMELINE and links libgdn_timeline.so); the product
// library compiles every mark to nothing.  Lane 0 of each wave writes the 100 MHz
// real-time counter at mark n into a device array indexed by (workgroup, wave, n),
// which gdn_timeline_read copies to the host.  Only workgroups below kTlGroups and
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
#define GDN_TL(n)                                                                                      \
    do {                                                                                               \
        const unsigned wg_ = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);          \
        if ((threadIdx.x & 63) == 0 && wg_ < (unsigned)gdn::kTlGroups && (threadIdx.x >> 6) < gdn::kTlWaves) \
            gdn::g_timeline[(wg_ * gdn::kTlWaves + (threadIdx.x >> 6)) * gdn::kTlMarks + (n)] =         \
                __builtin_amdgcn_s_memrealtime();                                                      \
    } while (0)
// the mark once value v is available (an empty asm statement that takes v: the wait for the load
// that produces v is placed before the mark)
#define GDN_TLV(n, v)                              \
    do {                                           \
        asm volatile("" ::"v"(v));                 \
        GDN_TL(n);                                 \
    } while (0)
#else
#define GDN_TL(n) ((void)0)
#define GDN_TLV(n, v) ((void)0)
#endif
