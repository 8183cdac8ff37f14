// Host-only stand-ins for the kernel launchers, so that the C ABI and the plan builder can
// be built without device code (for the host sanitizers).  They are reached only after a
// device was found; on a machine without one every launch path stops earlier.
#include "launch.h"

namespace wa {

hipError_t launch_forward(const ForwardArgs&, hipStream_t) { return hipErrorInvalidDevice; }
hipError_t launch_f32_to_bf16(const float*, void*, int64_t, hipStream_t) { return hipErrorInvalidDevice; }
hipError_t launch_qk_norm_rope(const PrologueArgs&, hipStream_t) { return hipErrorInvalidDevice; }
hipError_t launch_forward_fp8(const ForwardArgs&, float, hipStream_t) { return hipErrorInvalidDevice; }
hipError_t static_workspace(int, void**) { return hipErrorInvalidDevice; }

}  // namespace wa
