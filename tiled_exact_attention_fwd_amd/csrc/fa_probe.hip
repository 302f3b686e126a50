// Clock probe of include/fa_probe.h: shader cycles counted over a fixed
// stretch of real time, by one wave on each of 64 CUs.

#include <hip/hip_runtime.h>

#include "fa_fwd.h"
#include "fa_fwd_launch.h"
#include "fa_probe.h"

namespace {

// 64 single-wave workgroups, spread by the dispatcher over the CUs: each
// counts its CU's shader cycles over `ticks` ticks of the constant-rate
// real-time counter (a bounded wait: that counter always advances), and
// writes both counts.
__global__ void __launch_bounds__(64) clock_probe_kernel(unsigned long long* out, unsigned ticks) {
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    const unsigned long long c0 = __builtin_amdgcn_s_memtime();
    unsigned long long r1, c1;
    do {
        c1 = __builtin_amdgcn_s_memtime();
        r1 = __builtin_amdgcn_s_memrealtime();
    } while (r1 - r0 < ticks);
    if (threadIdx.x == 0) {
        *(__attribute__((address_space(1))) unsigned long long*)(out + 2 * blockIdx.x) = c1 - c0;
        *(__attribute__((address_space(1))) unsigned long long*)(out + 2 * blockIdx.x + 1) = r1 - r0;
    }
}

}  // namespace

extern "C" int fa_clock_probe(unsigned long long* out, unsigned ticks, void* stream) {
    if (!out || ticks == 0 || ticks > FA_PROBE_MAX_TICKS) return FA_ERR_INVALID;
    int cus = 0;
    const int st = fa::device_check(&cus);
    if (st != FA_OK) return st;
    hipLaunchKernelGGL(clock_probe_kernel, dim3(FA_PROBE_WAVES), dim3(64), 0, (hipStream_t)stream, out, ticks);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}
