// fa_launch.hpp -- launcher definitions; included by the shard files only.
#pragma once

#include "fa_fwd_kernel.hpp"
#include "fa_fwd_pair_kernel.hpp"
#include "fa_fwd_role_kernel.hpp"

namespace fa355 {

template <typename T, int D, int BC, int WAVES, bool CAUSAL, bool OUT_F32>
hipError_t launch_fwd(const FwdArgs &a, hipStream_t stream)
{
    using Tr = FwdTraits<T, D, BC, WAVES, CAUSAL, OUT_F32>;
    const void *fn = reinterpret_cast<const void *>(&fa_fwd_kernel<T, D, BC, WAVES, CAUSAL, OUT_F32>);
    FwdArgs arg = a;
    void *params[] = {&arg};
    return hipLaunchKernel(fn, dim3(a.total_tiles), dim3(Tr::NT), params, 0, stream);   // static LDS
}

template <typename T, int D, int BC, int WAVES, bool CAUSAL>
hipError_t launch_fwd_bias(const FwdArgs &a, hipStream_t stream)
{
    using Tr = FwdTraits<T, D, BC, WAVES, CAUSAL, false>;
    const void *fn = reinterpret_cast<const void *>(&fa_fwd_kernel<T, D, BC, WAVES, CAUSAL, false, false, true>);
    FwdArgs arg = a;
    void *params[] = {&arg};
    return hipLaunchKernel(fn, dim3(a.total_tiles), dim3(Tr::NT), params, 0, stream);   // static LDS
}

template <typename T, int D, int BC, int WAVES, bool CAUSAL>
hipError_t launch_fwd_split(const FwdArgs &a, hipStream_t stream)
{
    using Tr = FwdTraits<T, D, BC, WAVES, CAUSAL, false>;
    const void *fn = reinterpret_cast<const void *>(&fa_fwd_kernel<T, D, BC, WAVES, CAUSAL, false, true>);
    FwdArgs arg = a;
    void *params[] = {&arg};
    hipError_t e = hipLaunchKernel(fn, dim3(a.total_tiles * a.num_splits), dim3(Tr::NT), params,
                                   0, stream);   // static LDS
    if (e != hipSuccess)
        return e;
    const int64_t rows = (int64_t)a.B * a.Hq * a.N;
    constexpr int RPB = 256 / (D / 4);
    return hipLaunchKernel(reinterpret_cast<const void *>(&fa_fwd_merge_kernel<T, D>),
                           dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), params, 0, stream);
}

template <typename T, bool CAUSAL, bool OUT_F32>
hipError_t launch_fwd_pair(const FwdArgs &a, hipStream_t stream)
{
    const void *fn = reinterpret_cast<const void *>(&fa_fwd_pair_kernel<T, CAUSAL, OUT_F32>);
    FwdArgs arg = a;
    void *params[] = {&arg};
    return hipLaunchKernel(fn, dim3(a.total_tiles), dim3(PairTraits::NT), params, 0, stream);   // static LDS
}

template <typename T, bool CAUSAL, bool OUT_F32>
hipError_t launch_fwd_role(const FwdArgs &a, hipStream_t stream)
{
    const void *fn = reinterpret_cast<const void *>(&fa_fwd_role_kernel<T, CAUSAL, OUT_F32>);
    FwdArgs arg = a;
    void *params[] = {&arg};
    return hipLaunchKernel(fn, dim3(a.total_tiles), dim3(RoleTraits::NT), params, 0, stream);   // static LDS
}

template <int WAVES, bool CAUSAL>
hipError_t launch_fwd_f32(const FwdArgs &a, hipStream_t stream)
{
    using Tr = F32Traits<WAVES, CAUSAL>;
    const void *fn = reinterpret_cast<const void *>(&fa_fwd_f32_kernel<WAVES, CAUSAL>);
    FwdArgs arg = a;
    void *params[] = {&arg};
    return hipLaunchKernel(fn, dim3(a.total_tiles), dim3(Tr::NT), params, Tr::LDS, stream);
}

}  // namespace fa355

#define FA355_INSTANTIATE(T, D, BC, W, C, O)                                          \
    template hipError_t fa355::launch_fwd<fa355::T, D, BC, W, C, O>(const fa355::FwdArgs &, hipStream_t);
#define FA355_INSTANTIATE_PAIR(T, C, O)                                               \
    template hipError_t fa355::launch_fwd_pair<fa355::T, C, O>(const fa355::FwdArgs &, hipStream_t);
#define FA355_INSTANTIATE_ROLE(T, C, O)                                               \
    template hipError_t fa355::launch_fwd_role<fa355::T, C, O>(const fa355::FwdArgs &, hipStream_t);
#define FA355_INSTANTIATE_F32(W, C)                                                   \
    template hipError_t fa355::launch_fwd_f32<W, C>(const fa355::FwdArgs &, hipStream_t);
#define FA355_INSTANTIATE_SPLIT(T, D, BC, W, C)                                       \
    template hipError_t fa355::launch_fwd_split<fa355::T, D, BC, W, C>(const fa355::FwdArgs &, hipStream_t);
#define FA355_INSTANTIATE_BIAS(T, D, BC, W, C)                                        \
    template hipError_t fa355::launch_fwd_bias<fa355::T, D, BC, W, C>(const fa355::FwdArgs &, hipStream_t);
