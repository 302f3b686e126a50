// Tile-size sweep instances: bf16, d = 128, no mask, one (query rows, keys
// per tile) shape per translation unit, chosen by FA_TQ / FA_TK; the plain
// and the counting kernel of that shape, and its launcher.  A launch asks for
// one through fa_fwd_ex's tile_q / tile_k.

#include <hip/hip_runtime.h>

#include "fa_fwd_launch.h"

#if !defined(FA_TQ) || !defined(FA_TK)
#error "FA_TQ and FA_TK select the tile shape"
#endif

#define FA_CAT4(a, b, c, d) a##b##c##d
#define FA_XCAT4(a, b, c, d) FA_CAT4(a, b, c, d)

namespace fa {

int FA_XCAT4(launch16t_q, FA_TQ, _k, FA_TK)(const FwdParams& p, bool count, void* stream) {
    using Plain = Fwd16<BF16, 128, false, false, false, FA_TQ / 32, FA_TK>;
    using Count = Fwd16<BF16, 128, false, false, true, FA_TQ / 32, FA_TK>;
    static_assert(Plain::BQ == FA_TQ && Plain::BK == FA_TK, "tile shape");
    return count ? launch_kernel<Count>(p, stream) : launch_kernel<Plain>(p, stream);
}

}  // namespace fa
