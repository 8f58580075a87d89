// gdn_verify_f32_bf16.hip -- the verify kernel instances for f32 slabs and bf16 outputs (one
// translation unit per dtype pair, so the instances compile in parallel).
#include "gdn_verify_impl.h"

namespace gdn {

hipError_t launch_verify_f32_bf16(const VerifyArgs& a, hipStream_t s) { return launch_io<false, true>(a, s); }

}  // namespace gdn

GDN_CLAMP_READER(clamped_accepts_verify_f32_bf16)
