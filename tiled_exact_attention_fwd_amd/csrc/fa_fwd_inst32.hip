// The fp32 kernel instances of one mask setting (FA_INST_C) and their launcher.

#include <hip/hip_runtime.h>

#include "fa_fwd_launch.h"

#if !defined(FA_INST_C)
#error "FA_INST_C selects the instance"
#endif

#define FA_CAT2(a, b) a##b
#define FA_XCAT2(a, b) FA_CAT2(a, b)
#define FA_NAME FA_XCAT2(launch32_c, FA_INST_C)
#define FA_NAME_S FA_XCAT2(launch32s_c, FA_INST_C)

namespace fa {

int FA_NAME(const FwdParams& p, int d, bool count, void* stream) {
    constexpr bool C = FA_INST_C != 0;
    if (d == 64)
        return count ? launch_kernel<Fwd32<64, C, true>>(p, stream) : launch_kernel<Fwd32<64, C, false>>(p, stream);
    return count ? launch_kernel<Fwd32<128, C, true>>(p, stream) : launch_kernel<Fwd32<128, C, false>>(p, stream);
}

// split-KV: fp32 partials over key ranges, then the merge (fp32 output)
int FA_NAME_S(const FwdParams& p, int d, void* o, float* lse, void* stream) {
    constexpr bool C = FA_INST_C != 0;
    void* args[] = {const_cast<FwdParams*>(&p)};
    const void* k64 = (const void*)&fwd_kernel<Fwd32<64, C, false, true>>;
    const void* k128 = (const void*)&fwd_kernel<Fwd32<128, C, false, true>>;
    hipError_t err = hipLaunchKernel(d == 64 ? k64 : k128, dim3(p.total * p.splits), dim3(Fwd32<64, C, false>::NT),
                                     args, 0, (hipStream_t)stream);
    if (err != hipSuccess) return FA_ERR_HIP;
    const int rows = p.heads * p.N;
    if (d == 64)
        hipLaunchKernelGGL((split_merge_kernel<float, 64>), dim3((rows + 31) / 32), dim3(256), 0, (hipStream_t)stream,
                           (const float*)p.o, (const float*)p.lse, o, lse, rows, p.splits);
    else
        hipLaunchKernelGGL((split_merge_kernel<float, 128>), dim3((rows + 15) / 16), dim3(256), 0,
                           (hipStream_t)stream, (const float*)p.o, (const float*)p.lse, o, lse, rows, p.splits);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace fa
