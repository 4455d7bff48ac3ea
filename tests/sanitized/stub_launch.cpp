// Host-only stand-ins for the kernel launchers of libsage, for the sanitised
// build of the C-ABI front end (sage_abi.hip) that runs the host ABI tests on
// a machine without a GPU. Each launcher reports what the HIP runtime reports
// there (no device), so the front end behaves exactly as the real library does
// on such a machine; the front end's own validation, workspace arithmetic and
// aliasing checks are what the sanitisers watch.
#include "sage_launch.h"

namespace sage {

hipError_t launch_varlen_plan(const int32_t*, const int32_t*, int, int, int, int, int, int, SeqSpan*, int32_t*, int,
                              hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_quant_qk(const QuantQKArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_quant_v(const QuantVArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_attn(const AttnArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_debug_qk(const DebugQKArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_k_mean(const void*, TensorGeom, int, int, int, int, bool, double*, float*, hipStream_t,
                         const SeqSpan*) {
  return hipErrorNoDevice;
}
hipError_t launch_quant_fp4(const Fp4QuantArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_attn_fp4(const Fp4AttnArgs&, hipStream_t) { return hipErrorNoDevice; }

}  // namespace sage
