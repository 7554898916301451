// Fused differential-attention forward, the launches: the kernels and their design are in
// fwd_mfma_kernel.hpp. This file builds them under the compiler's default instruction schedule
// and serves keys shorter than kLongKeys; fwd_mfma_long.hip builds the same kernels under the
// max-ilp schedule for longer ones (measured on MI355X, outputs bit-identical: max-ilp 0.8% slower
// at 2K keys, 0.8% faster at 4K, 1.0% at 8K, 1.4% at 32K, 1.6% for the V2 8K GQA prefill).
#include "fwd_mfma_kernel.hpp"

namespace diffattn {

hipError_t launch_v1_fwd_mfma(const MfmaFwdArgs& a, hipStream_t stream) {
    return a.seq_k >= kLongKeys ? launch_v1_fwd_mfma_long(a, stream) : launch_fwd<64, false>(a, stream);
}
hipError_t launch_v2_fwd_mfma(const MfmaFwdArgs& a, hipStream_t stream) {
    return a.seq_k >= kLongKeys ? launch_v2_fwd_mfma_long(a, stream) : launch_fwd<128, true>(a, stream);
}
hipError_t launch_v1_fwd_fp8(const MfmaFwdArgs& a, hipStream_t stream) {
    return a.seq_k >= kLongKeys ? launch_v1_fwd_fp8_long(a, stream) : launch_fwd<64, false, true>(a, stream);
}

}  // namespace diffattn
