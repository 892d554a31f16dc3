// Launcher stand-ins for the host-only sanitizer build of fa_api.hip: the
// validation and dispatch code runs unchanged, and a call that passes every
// check ends here instead of launching a kernel (no GPU code is built).
#include "fa_launch.h"

namespace fa {
hipError_t launch_fwd_bf16(const FwdArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_bwd_bf16(const BwdArgs&, unsigned, hipStream_t) { return hipSuccess; }
hipError_t launch_fwd_f32(const FwdArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_bwd_f32(const BwdArgs&, unsigned, hipStream_t) { return hipSuccess; }
hipError_t launch_splitkv_bf16(const SplitKvArgs&, unsigned, hipStream_t) { return hipSuccess; }
}  // namespace fa
