// fp32 backward kernel instances (d = 64 and 128, both mask settings) and
// their launcher.

#include <hip/hip_runtime.h>

#include "fa_bwd32_kernels.h"
#include "fa_bwd_launch.h"

namespace fa {
namespace bwd {

namespace {
template <int D, bool C>
int launch32(const BwdParams32& p, int heads, void* stream) {
    const dim3 grid((unsigned)(heads * p.nblk)), block(256);
    const hipStream_t st = (hipStream_t)stream;
    hipLaunchKernelGGL((dq_kernel32<D, C>), grid, block, 0, st, p);
    hipLaunchKernelGGL((dkdv_kernel32<D, C>), grid, block, 0, st, p);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}
}  // namespace

int launch_bwd_f32(const BwdParams32& p, int heads, int d, bool causal, void* stream) {
    if (d == 64) return causal ? launch32<64, true>(p, heads, stream) : launch32<64, false>(p, heads, stream);
    return causal ? launch32<128, true>(p, heads, stream) : launch32<128, false>(p, heads, stream);
}

}  // namespace bwd
}  // namespace fa
