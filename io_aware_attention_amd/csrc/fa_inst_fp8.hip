// Forward kernels with e4m3 inputs: head dims 64 and 128, causal and not.
#include "fa_fp8_kernel.hpp"

namespace fa355 {
template <int D, bool CAUSAL>
hipError_t launch_fwd_fp8(const FwdArgs &a, hipStream_t stream)
{
    return launch_fwd_fp8_impl<D, CAUSAL>(a, stream);
}
template hipError_t launch_fwd_fp8<64, false>(const FwdArgs &, hipStream_t);
template hipError_t launch_fwd_fp8<64, true>(const FwdArgs &, hipStream_t);
template hipError_t launch_fwd_fp8<128, false>(const FwdArgs &, hipStream_t);
template hipError_t launch_fwd_fp8<128, true>(const FwdArgs &, hipStream_t);
}  // namespace fa355
