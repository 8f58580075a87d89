// gdn_debug.h -- the debug build's count of clamped accept lengths.
//
// An accept length outside the range of the window it refers to (0..K) is
// clamped by every kernel that reads one; the debug build (GDN_DEBUG,
// libgdn_debug.so) also counts it, once per sequence and call, so a caller's
// off-by-one shows up as a number instead of a silently shortened rollback.
// The release build compiles none of this.
//
// There is no relocatable device code, so each translation unit that clamps
// has a counter of its own and a host reader (GDN_CLAMP_READER); the ABI call
// gdn_debug_clamped_accepts sums them.
#pragma once

#include <hip/hip_runtime.h>

#ifdef GDN_DEBUG
namespace gdn {
static __device__ unsigned long long g_clamped_accepts;
}  // namespace gdn
// the caller evaluates `cond` in one thread per sequence
#define GDN_COUNT_CLAMP(cond)                                                                        \
    do {                                                                                             \
        if (cond) atomicAdd(&gdn::g_clamped_accepts, 1ull);                                          \
    } while (0)
// NAME(n, reset): this translation unit's count into *n (host), then zero if reset
#define GDN_CLAMP_READER(NAME)                                                                       \
    namespace gdn {                                                                                  \
    hipError_t NAME(unsigned long long* n, bool reset)                                               \
    {                                                                                                \
        hipError_t e = hipMemcpyFromSymbol(n, HIP_SYMBOL(g_clamped_accepts), sizeof(*n), 0,          \
                                           hipMemcpyDeviceToHost);                                   \
        if (e == hipSuccess && reset) {                                                              \
            const unsigned long long z = 0;                                                          \
            e = hipMemcpyToSymbol(HIP_SYMBOL(g_clamped_accepts), &z, sizeof(z), 0,                   \
                                  hipMemcpyHostToDevice);                                            \
        }                                                                                            \
        return e;                                                                                    \
    }                                                                                                \
    }
#else
#define GDN_COUNT_CLAMP(cond) \
    do {                      \
    } while (0)
#define GDN_CLAMP_READER(NAME)
#endif
