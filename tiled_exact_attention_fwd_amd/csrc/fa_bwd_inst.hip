// Backward kernel instances of one element type and head dimension
// (FA_INST_T, FA_INST_D), both mask settings, and their launcher.

#include <hip/hip_runtime.h>

#include "fa_bwd_kernels.h"
#include "fa_bwd_launch.h"

#if !defined(FA_INST_T) || !defined(FA_INST_D)
#error "FA_INST_T and FA_INST_D select the instance"
#endif

#define FA_CAT4(a, b, c, d) a##b##c##d
#define FA_XCAT4(a, b, c, d) FA_CAT4(a, b, c, d)
#define FA_NAME FA_XCAT4(launch_bwd_, FA_INST_T, _d, FA_INST_D)

namespace fa {
namespace bwd {

namespace {
struct bf16 { using T = BF16; };
struct f16 { using T = F16; };

template <class T, int D, bool C, bool O32>
int launch(const BwdParams& p0, int heads, int cus, void* stream) {
    BwdParams p = p0;
    p.nblk = (p.N + DqShape<D>::ROWS - 1) / DqShape<D>::ROWS;
    p.nblk_k = (p.N + DkdvShape<D>::KEYS - 1) / DkdvShape<D>::KEYS;
    // causal: heads per group as in the forward (a group's blocks fill the
    // XCD's workgroup slots twice)
    p.group = causal_group(heads, p.nblk, cus / kNumXcd * DqShape<D>::PER_CU);
    p.group_k = causal_group(heads, p.nblk_k, cus / kNumXcd * DkdvShape<D>::PER_CU);
    const hipStream_t st = (hipStream_t)stream;
    hipLaunchKernelGGL((dq_kernel<T, D, C, O32>), dim3((unsigned)(heads * p.nblk)), dim3(DqShape<D>::NT), 0, st, p);
    hipLaunchKernelGGL((dkdv_kernel<T, D, C>), dim3((unsigned)(heads * p.nblk_k)), dim3(DkdvShape<D>::NT), 0, st, p);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}
}  // namespace

int FA_NAME(const BwdParams& p, int heads, int cus, bool causal, void* stream) {
    using T = FA_INST_T::T;
    if (p.o32)
        return causal ? launch<T, FA_INST_D, true, true>(p, heads, cus, stream)
                      : launch<T, FA_INST_D, false, true>(p, heads, cus, stream);
    return causal ? launch<T, FA_INST_D, true, false>(p, heads, cus, stream)
                  : launch<T, FA_INST_D, false, false>(p, heads, cus, stream);
}

}  // namespace bwd
}  // namespace fa
