// The fp32 kernel instances of one mask setting (FA_INST_C) and their launcher.

#include <hip/hip_runtime.h>

#include "fa_fwd_launch.h"

#if !defined(FA_INST_C)
#error "FA_INST_C selects the instance"
#endif

#define FA_CAT2(a, b) a##b
#define FA_XCAT2(a, b) FA_CAT2(a, b)
#define FA_NAME FA_XCAT2(launch32_c, FA_INST_C)

namespace fa {

int FA_NAME(const FwdParams& p, int d, bool count, void* stream) {
    constexpr bool C = FA_INST_C != 0;
    if (d == 64)
        return count ? launch_kernel<Fwd32<64, C, true>>(p, stream) : launch_kernel<Fwd32<64, C, false>>(p, stream);
    return count ? launch_kernel<Fwd32<128, C, true>>(p, stream) : launch_kernel<Fwd32<128, C, false>>(p, stream);
}

}  // namespace fa
