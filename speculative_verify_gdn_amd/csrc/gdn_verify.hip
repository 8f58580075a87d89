// gdn_verify.hip -- dispatch of the verify kernel (gdn_verify_impl.h) by input and output dtype.
#include "gdn_internal.h"

namespace gdn {

hipError_t launch_verify_bf16_f32(const VerifyArgs& a, hipStream_t s);
hipError_t launch_verify_bf16_bf16(const VerifyArgs& a, hipStream_t s);
hipError_t launch_verify_f32_f32(const VerifyArgs& a, hipStream_t s);
hipError_t launch_verify_f32_bf16(const VerifyArgs& a, hipStream_t s);

hipError_t launch_verify(const VerifyArgs& a, bool in_bf16, bool o_bf16, hipStream_t s)
{
    if (in_bf16) return o_bf16 ? launch_verify_bf16_bf16(a, s) : launch_verify_bf16_f32(a, s);
    return o_bf16 ? launch_verify_f32_bf16(a, s) : launch_verify_f32_f32(a, s);
}

}  // namespace gdn
