// fa_bwd_launch.hpp -- backward launcher definitions; included by the shard files.
#pragma once

#include "fa_bwd_kernel.hpp"

namespace fa355 {

template <typename T, int D, bool CAUSAL>
hipError_t launch_bwd(const BwdArgs &a, hipStream_t stream)
{
    BwdArgs arg = a;
    void *params[] = {&arg};
    const int64_t rows = (int64_t)a.B * a.Hq * a.N;
    constexpr int RPB = 256 / (D / 8);
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&fa_bwd_delta_kernel<T, D>),
                                   dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), params, 0, stream);
    if (e != hipSuccess)
        return e;
    e = hipLaunchKernel(reinterpret_cast<const void *>(&fa_bwd_dkdv_role_kernel<T, D, CAUSAL>),
                        dim3(a.B * a.Hkv * a.n_ktiles), dim3(512), params, 0, stream);
    if (e != hipSuccess)
        return e;
    if constexpr (D != 256) {
        if (a.dq_rows == 256)
            return hipLaunchKernel(reinterpret_cast<const void *>(&fa_bwd_dq_kernel<T, D, CAUSAL, 8>),
                                   dim3(a.total_tiles), dim3(512), params, 0, stream);
    }
    if (a.dq_rows != 128)
        return hipErrorInvalidValue;
    return hipLaunchKernel(reinterpret_cast<const void *>(&fa_bwd_dq_kernel<T, D, CAUSAL, 4>),
                           dim3(a.total_tiles), dim3(256), params, 0, stream);
}

}  // namespace fa355

#define FA355_INSTANTIATE_BWD(T, D, C)                                                \
    template hipError_t fa355::launch_bwd<fa355::T, D, C>(const fa355::BwdArgs &, hipStream_t);
