// gdn_verify_f32_f32.hip -- the verify kernel instances for f32 slabs and f32 outputs (one
// translation unit per dtype pair, so the instances compile in parallel).
#include "gdn_verify_impl.h"

namespace gdn {

hipError_t launch_verify_f32_f32(const VerifyArgs& a, hipStream_t s) { return launch_io<false, false>(a, s); }

}  // namespace gdn

GDN_CLAMP_READER(clamped_accepts_verify_f32_f32)
