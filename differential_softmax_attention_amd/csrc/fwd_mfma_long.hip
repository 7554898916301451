// The fused forward's kernels (fwd_mfma_kernel.hpp) built under the max-ilp instruction schedule
// (the build gives this file -amdgpu-sched-strategy=max-ilp), for keys of kLongKeys and more.
#include "fwd_mfma_kernel.hpp"

namespace diffattn {

hipError_t launch_v1_fwd_mfma_long(const MfmaFwdArgs& a, hipStream_t stream) { return launch_fwd<64, false>(a, stream); }
hipError_t launch_v2_fwd_mfma_long(const MfmaFwdArgs& a, hipStream_t stream) { return launch_fwd<128, true>(a, stream); }
hipError_t launch_v1_fwd_fp8_long(const MfmaFwdArgs& a, hipStream_t stream) { return launch_fwd<64, false, true>(a, stream); }

}  // namespace diffattn
