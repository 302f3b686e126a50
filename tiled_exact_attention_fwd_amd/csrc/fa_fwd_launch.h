// Kernel-instance launchers of the forward library.  Each is defined in its
// own translation unit (fa_fwd_inst16.hip / fa_fwd_inst32.hip compiled once
// per instance) so the instances build in parallel; the host layer
// (fa_fwd.hip) picks one after its argument checks.  All return an fa_status.
#pragma once

#include "fa_fwd.h"
#include "fa_fwd_kernels.h"

namespace fa {

// Query rows per workgroup of the per-tile 16-bit kernels (the same for
// both element types); the host sizes the grid with it.
constexpr int tile_q16(bool causal, int d) {
    return d == 64 ? (causal ? Fwd16<BF16, 64, true, false, false>::BQ : Fwd16<BF16, 64, false, false, false>::BQ)
                   : (causal ? Fwd16<BF16, 128, true, false, false>::BQ : Fwd16<BF16, 128, false, false, false>::BQ);
}
// Workgroups of one per-tile kernel resident on a CU at a time (the causal
// tile order groups heads by it)
constexpr int resident16(bool causal, int d) {
    return d == 64 ? (causal ? Fwd16<BF16, 64, true, false, false>::RESIDENT
                             : Fwd16<BF16, 64, false, false, false>::RESIDENT)
                   : (causal ? Fwd16<BF16, 128, true, false, false>::RESIDENT
                             : Fwd16<BF16, 128, false, false, false>::RESIDENT);
}
constexpr int resident32() { return Fwd32<64, true, false>::RESIDENT; }

#define FA_DECLARE16(T, D, C) \
    int launch16_##T##_d##D##_c##C(const FwdParams& p, int out_f32, bool count, void* stream);
FA_DECLARE16(bf16, 64, 0)
FA_DECLARE16(bf16, 64, 1)
FA_DECLARE16(bf16, 128, 0)
FA_DECLARE16(bf16, 128, 1)
FA_DECLARE16(f16, 64, 0)
FA_DECLARE16(f16, 64, 1)
FA_DECLARE16(f16, 128, 0)
FA_DECLARE16(f16, 128, 1)
#undef FA_DECLARE16
// persistent kernels (d = 128, no mask, 16-bit output; at least
// persistent_min_key_tiles() key tiles), launched on `grid` workgroups (one
// per CU); count selects the instrumented instance
int launch16p_bf16_d128(const FwdParams& p, int grid, bool count, void* stream);
int launch16p_f16_d128(const FwdParams& p, int grid, bool count, void* stream);
constexpr int persistent_tile_q() { return Fwd16P<BF16, 128>::BQ; }
constexpr int persistent_min_key_tiles() { return Fwd16P<BF16, 128>::MIN_KEY_TILES; }
// causal persistent kernels with 256-row query tiles (d = 128; an even number
// of query tiles, paired; every query tile at least 4 key tiles)
constexpr int wide_tile_q() { return Fwd16P<BF16, 128, true, true>::BQ; }
int launch16pcw_bf16_d128(const FwdParams& p, int grid, bool count, void* stream);
int launch16pcw_f16_d128(const FwdParams& p, int grid, bool count, void* stream);
// split-KV launches: p.o / p.lse point at the fp32 partials ([p.splits,
// B H, N] x d and [p.splits, B H, N]); the merge writes o and lse
#define FA_DECLARE16S(T, D, C) \
    int launch16s_##T##_d##D##_c##C(const FwdParams& p, void* o, float* lse, void* stream);
FA_DECLARE16S(bf16, 64, 0)
FA_DECLARE16S(bf16, 64, 1)
FA_DECLARE16S(bf16, 128, 0)
FA_DECLARE16S(bf16, 128, 1)
FA_DECLARE16S(f16, 64, 0)
FA_DECLARE16S(f16, 64, 1)
FA_DECLARE16S(f16, 128, 0)
FA_DECLARE16S(f16, 128, 1)
#undef FA_DECLARE16S
// tile-size sweep (bf16, d = 128, no mask): every (query rows, keys) in
// {64, 128, 256} x {32, 64, 128} besides the default 256 x 64
#define FA_DECLARE_TILE(Q, K) int launch16t_q##Q##_k##K(const FwdParams& p, bool count, void* stream);
FA_DECLARE_TILE(64, 32)
FA_DECLARE_TILE(64, 64)
FA_DECLARE_TILE(64, 128)
FA_DECLARE_TILE(128, 32)
FA_DECLARE_TILE(128, 64)
FA_DECLARE_TILE(128, 128)
FA_DECLARE_TILE(256, 32)
FA_DECLARE_TILE(256, 128)
#undef FA_DECLARE_TILE
int launch32_c0(const FwdParams& p, int d, bool count, void* stream);
int launch32_c1(const FwdParams& p, int d, bool count, void* stream);
// fp32 split-KV (partials and merge; 64-row query tiles)
int launch32s_c0(const FwdParams& p, int d, void* o, float* lse, void* stream);
int launch32s_c1(const FwdParams& p, int d, void* o, float* lse, void* stream);

// The current device: FA_OK if it is a gfx950 (and its compute-unit count
// in *cus), FA_ERR_UNSUPPORTED otherwise, FA_ERR_HIP if the query fails.
// Cached per device; shared by every host layer of the library.
int device_check(int* cus);

// launch of one kernel instance on the caller's stream
// (one workgroup per query tile, or `grid` workgroups for a persistent kernel)
template <class K>
int launch_kernel(const FwdParams& p, void* stream, int grid = 0) {
    void* args[] = {const_cast<FwdParams*>(&p)};
    const hipError_t err = hipLaunchKernel((const void*)&fwd_kernel<K>, dim3(grid > 0 ? grid : p.total), dim3(K::NT),
                                          args, 0, (hipStream_t)stream);
    return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace fa
