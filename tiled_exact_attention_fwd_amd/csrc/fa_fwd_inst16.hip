// One 16-bit kernel instance family (element type, head dimension, causal),
// chosen by FA_INST_T / FA_INST_D / FA_INST_C at compile time: the fp32-output
// and counter variants of it, and its launcher.

#include <hip/hip_runtime.h>

#include "fa_fwd_launch.h"

#if !defined(FA_INST_T) || !defined(FA_INST_D) || !defined(FA_INST_C)
#error "FA_INST_T, FA_INST_D and FA_INST_C select the instance"
#endif

#define FA_CAT6(a, b, c, d, e, f) a##b##c##d##e##f
#define FA_XCAT6(a, b, c, d, e, f) FA_CAT6(a, b, c, d, e, f)
#define FA_NAME FA_XCAT6(launch16_, FA_INST_T, _d, FA_INST_D, _c, FA_INST_C)
#define FA_TYPE_bf16 BF16
#define FA_TYPE_f16 F16
#define FA_TYPE_(t) FA_TYPE_##t
#define FA_TYPE(t) FA_TYPE_(t)

namespace fa {

int FA_NAME(const FwdParams& p, int out_f32, bool count, void* stream) {
    using T = FA_TYPE(FA_INST_T);
    constexpr bool C = FA_INST_C != 0;
    static_assert(Fwd16<T, FA_INST_D, C, true, true>::BQ == tile_q16(C, FA_INST_D), "grid tile");
    if (out_f32)
        return count ? launch_kernel<Fwd16<T, FA_INST_D, C, true, true>>(p, stream)
                     : launch_kernel<Fwd16<T, FA_INST_D, C, true, false>>(p, stream);
    return count ? launch_kernel<Fwd16<T, FA_INST_D, C, false, true>>(p, stream)
                 : launch_kernel<Fwd16<T, FA_INST_D, C, false, false>>(p, stream);
}

// split-KV: partials over key ranges (per-tile kernel, fp32 output), then the merge
int FA_XCAT6(launch16s_, FA_INST_T, _d, FA_INST_D, _c, FA_INST_C)(const FwdParams& p, void* o, float* lse,
                                                                   void* stream) {
    using K = Fwd16<FA_TYPE(FA_INST_T), FA_INST_D, FA_INST_C != 0, true, false, 0, 64, true>;
    static_assert(K::BQ == tile_q16(FA_INST_C != 0, FA_INST_D) && K::BK == 64, "grid tile");
    void* args[] = {const_cast<FwdParams*>(&p)};
    hipError_t err = hipLaunchKernel((const void*)&fwd_kernel<K>, dim3(p.total * p.splits), dim3(K::NT), args, 0,
                                     (hipStream_t)stream);
    if (err != hipSuccess) return FA_ERR_HIP;
    const int rows = p.heads * p.N;
    constexpr int rows_per_block = 256 / (FA_INST_D / 8);
    hipLaunchKernelGGL((split_merge_kernel<FA_TYPE(FA_INST_T), FA_INST_D>),
                       dim3((rows + rows_per_block - 1) / rows_per_block), dim3(256), 0,
                       (hipStream_t)stream, (const float*)p.o, (const float*)p.lse, o, lse, rows, p.splits);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

#define FA_CAT4(a, b, c, d) a##b##c##d
#define FA_XCAT4(a, b, c, d) FA_CAT4(a, b, c, d)
#if FA_INST_D == 128 && FA_INST_C == 0
// the persistent kernel (no mask, 16-bit output) on `grid` workgroups; count:
// its instrumented instance
int FA_XCAT4(launch16p_, FA_INST_T, _d, FA_INST_D)(const FwdParams& p, int grid, bool count, void* stream) {
    using K = Fwd16P<FA_TYPE(FA_INST_T), FA_INST_D>;
    static_assert(K::BQ == persistent_tile_q(), "grid tile");
    return count ? launch_kernel<Fwd16PCount<FA_TYPE(FA_INST_T), FA_INST_D>>(p, stream, grid)
                 : launch_kernel<K>(p, stream, grid);
}
#elif FA_INST_D == 128
// the causal persistent kernel with 256-row query tiles (d = 128, 16-bit
// output); count: its instrumented instance
int FA_XCAT4(launch16pcw_, FA_INST_T, _d, FA_INST_D)(const FwdParams& p, int grid, bool count, void* stream) {
    static_assert(Fwd16P<FA_TYPE(FA_INST_T), FA_INST_D, true, true>::BQ == wide_tile_q(), "grid tile");
    return count ? launch_kernel<Fwd16PCount<FA_TYPE(FA_INST_T), FA_INST_D, true, true>>(p, stream, grid)
                 : launch_kernel<Fwd16P<FA_TYPE(FA_INST_T), FA_INST_D, true, true>>(p, stream, grid);
}
#endif

}  // namespace fa
