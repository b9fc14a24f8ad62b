// Decoding kernels: 16-bit inputs, head dims 64 and 128, causal and not.
#include "fa_decode_kernel.hpp"

namespace fa355 {
template <typename T, int D, bool CAUSAL>
hipError_t launch_decode(const DecodeArgs &a, const FwdArgs &merge, hipStream_t stream)
{
    DecodeArgs arg = a;
    void *params[] = {&arg};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&fa_decode_kernel<T, D, CAUSAL>),
                                   dim3(a.B * a.Hkv * a.num_splits), dim3(64), params, 0, stream);
    if (e != hipSuccess)
        return e;
    FwdArgs m = merge;
    void *mparams[] = {&m};
    const int64_t rows = (int64_t)m.B * m.Hq * m.N;
    return hipLaunchKernel(reinterpret_cast<const void *>(&fa_decode_merge_kernel<T, D>),
                           dim3((unsigned)rows, D / 32), dim3(256), mparams, 0, stream);
}
#define FA355_INST_DECODE(T, D, C) \
    template hipError_t launch_decode<T, D, C>(const DecodeArgs &, const FwdArgs &, hipStream_t);
FA355_INST_DECODE(BF16, 64, false) FA355_INST_DECODE(BF16, 64, true)
FA355_INST_DECODE(BF16, 128, false) FA355_INST_DECODE(BF16, 128, true)
FA355_INST_DECODE(F16, 64, false) FA355_INST_DECODE(F16, 64, true)
FA355_INST_DECODE(F16, 128, false) FA355_INST_DECODE(F16, 128, true)
}  // namespace fa355
