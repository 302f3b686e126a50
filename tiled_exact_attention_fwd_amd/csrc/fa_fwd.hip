// Host layer of the C ABI declared in include/fa_fwd.h: argument checks (all
// before any HIP call), kernel-instance selection, launch on the caller's
// stream.  No allocation, no synchronisation, no printing.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cfloat>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "fa_fwd.h"
#include "fa_fwd_launch.h"

#ifndef FA_BUILD_FLAGS
#define FA_BUILD_FLAGS "unknown"
#endif

namespace {

using fa::BF16;
using fa::F16;
using fa::FwdParams;

constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other
std::atomic<int> g_dev_cus[kMaxDevices];     // compute units, once known

int elem_size(int dtype) { return dtype == FA_DTYPE_F32 ? 4 : 2; }

bool overlaps(const void* a, uint64_t an, const void* b, uint64_t bn) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bn && b0 < a0 + an;
}

// Default tile shape per element type, head dimension and mask.
void tile_shape(int dtype, int d, int causal, int* tq, int* tk) {
    if (dtype == FA_DTYPE_F32) { *tq = 64; *tk = 64; }
    else { *tq = fa::tile_q16(causal != 0, d); *tk = 64; }
}

// The tile-size sweep shapes: bf16, d = 128, no mask, 16-bit output,
// (query rows, keys) in {64, 128, 256} x {32, 64, 128}.
bool sweep_shape(const fa_fwd_args* a, int tq, int tk) {
    return a->dtype == FA_DTYPE_BF16 && a->d == 128 && !a->causal && !a->out_dtype &&
           (tq == 64 || tq == 128 || tq == 256) && (tk == 32 || tk == 64 || tk == 128);
}

// The shape a launch uses: the default, or the one it asks for.
int launch_shape(const fa_fwd_args* a, int* tq, int* tk) {
    tile_shape(a->dtype, a->d, a->causal, tq, tk);
    if (a->tile_q < 0 || a->tile_k < 0) return FA_ERR_INVALID;
    const int rq = a->tile_q ? a->tile_q : *tq, rk = a->tile_k ? a->tile_k : *tk;
    if ((rq != *tq || rk != *tk) && !sweep_shape(a, rq, rk)) return FA_ERR_UNSUPPORTED;
    *tq = rq;
    *tk = rk;
    return FA_OK;
}

int check_args(const fa_fwd_args* a) {
    if (!a) return FA_ERR_INVALID;
    if (a->B <= 0 || a->H <= 0 || a->N <= 0 || a->d <= 0) return FA_ERR_INVALID;
    if (!a->q || !a->k || !a->v || !a->o || !a->lse) return FA_ERR_INVALID;
    if (a->causal != 0 && a->causal != 1) return FA_ERR_INVALID;
    if (!std::isfinite(a->scale)) return FA_ERR_INVALID;
    if (a->out_dtype != 0 && a->out_dtype != 1) return FA_ERR_INVALID;
    if (a->dtype != FA_DTYPE_F32 && a->dtype != FA_DTYPE_F16 && a->dtype != FA_DTYPE_BF16)
        return FA_ERR_UNSUPPORTED;
    if (a->d != 64 && a->d != 128) return FA_ERR_UNSUPPORTED;
    int tq, tk;
    const int ts = launch_shape(a, &tq, &tk);
    if (ts != FA_OK) return ts;
    const int e = elem_size(a->dtype);
    if ((uint64_t)a->N * a->d * 4 >= (1ull << 31)) return FA_ERR_UNSUPPORTED;   // per-head bytes
    const uint64_t tiles = (uint64_t)a->B * a->H * (uint64_t)((a->N + tq - 1) / tq);
    if (tiles >= (1ull << 31)) return FA_ERR_UNSUPPORTED;
    const uint64_t elems = (uint64_t)a->B * a->H * a->N * a->d;
    const uint64_t in_b = elems * e;
    const uint64_t out_b = elems * (a->out_dtype ? 4 : e);
    const uint64_t lse_b = (uint64_t)a->B * a->H * a->N * 4;
    const void* ins[3] = {a->q, a->k, a->v};
    for (const void* in : ins) {
        if (overlaps(a->o, out_b, in, in_b)) return FA_ERR_INVALID;
        if (overlaps(a->lse, lse_b, in, in_b)) return FA_ERR_INVALID;
    }
    if (overlaps(a->o, out_b, a->lse, lse_b)) return FA_ERR_INVALID;
    return FA_OK;
}

int check_device(int* cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
    int st = g_dev_state[dev].load(std::memory_order_acquire);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FA_ERR_HIP;
        st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_dev_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
        g_dev_state[dev].store(st, std::memory_order_release);
    }
    *cus = g_dev_cus[dev].load(std::memory_order_relaxed);
    return st == 1 ? FA_OK : FA_ERR_UNSUPPORTED;
}

// The kernel a launch runs, chosen from the arguments and the device's
// compute units; a launch with tile counters takes the same choice (the
// instrumented instance of the same kernel), so its counts are those of the
// kernel the plain launch runs.
enum LaunchKind { kSweep, kPersistent, kPersistentCausalWide, kPerTile16, kPerTile32 };
struct LaunchPlan {
    LaunchKind kind;
    int tq, tk;     // query rows and keys of the tile the kernel works in
    int grid;       // workgroups of a persistent kernel (0: one per query tile)
};

LaunchPlan plan_launch(const fa_fwd_args* a, int cus) {
    int tq, tk;
    launch_shape(a, &tq, &tk);
    const bool c = a->causal != 0, o32 = a->out_dtype != 0, f32 = a->dtype == FA_DTYPE_F32;
    if (f32) return {kPerTile32, tq, tk, 0};
    // an explicitly requested tile-size sweep shape: the per-tile kernel of
    // that shape (for the default shape too, so that a sweep compares one
    // kernel family)
    if (a->tile_q && sweep_shape(a, tq, tk)) return {kSweep, tq, tk, 0};
    const long long heads = (long long)a->B * a->H;
    // A 16-bit launch at d = 128 without a mask that has more query tiles
    // than the device has CUs runs the persistent kernel: one workgroup per
    // CU (a multiple of 8, so that each keeps to one XCD's tiles) takes every
    // slots-th query tile and pipelines across them.  (At d = 64 three
    // per-tile workgroups share a CU and keep it as busy; a persistent kernel
    // with three workgroups per CU measured 1-2% either side of them.)
    const int slots = cus / fa::kNumXcd * fa::kNumXcd;
    const int nk = (a->N + tk - 1) / tk;
    const long long tiles = heads * ((a->N + tq - 1) / tq);
    if (!c && a->d == 128 && !o32 && slots > 0 && tiles > slots && nk >= fa::persistent_min_key_tiles())
        return {kPersistent, fa::persistent_tile_q(), tk, slots};
    // Under the causal mask at d = 128: the persistent kernel with 256-row
    // query tiles (one workgroup per CU), each work unit a pair of query
    // tiles (i, T - 1 - i) of one head, whose key tiles add up to the same
    // count for every pair; the shortest tile must have 4 key tiles.
    if (c && a->d == 128 && !o32 && slots > 0) {
        const int tw = fa::wide_tile_q(), wtiles = (a->N + tw - 1) / tw;
        const int nk_first = (std::min(tw, a->N) - 1) / tk + 1;
        if (wtiles % 2 == 0 && nk_first >= 4 && heads * wtiles / 2 > slots)
            return {kPersistentCausalWide, tw, tk, slots};
    }
    return {kPerTile16, tq, tk, 0};
}

int run(const fa_fwd_args* a) {
    int st = check_args(a);
    if (st != FA_OK) return st;
    int cus = 0;
    st = check_device(&cus);
    if (st != FA_OK) return st;

    const LaunchPlan plan = plan_launch(a, cus);
    FwdParams p;
    p.q = a->q;
    p.k = a->k;
    p.v = a->v;
    p.o = a->o;
    p.lse = a->lse;
    p.N = a->N;
    p.tiles_q = (a->N + plan.tq - 1) / plan.tq;
    p.heads = a->B * a->H;
    p.total = p.heads * p.tiles_q;
    const int resident = a->dtype == FA_DTYPE_F32 ? fa::resident32() : fa::resident16(a->causal != 0, a->d);
    p.group = a->dtype == FA_DTYPE_F32 ? fa::causal_group(p.heads, p.tiles_q, cus / fa::kNumXcd * resident)
                                        : fa::fwd_causal_group(p.heads);
    // softmax in base 2: exp(scale * s) = 2^(s * |scale| * log2 e) after a sign
    // flip of Q for negative scales; FLT_MIN keeps -inf * c at -inf for scale 0
    p.c = std::fmax(std::fabs(a->scale) * 1.4426950408889634f, FLT_MIN);
    const bool neg = a->scale < 0.f;
    p.qsign = neg ? (a->dtype == FA_DTYPE_F32 ? 0x80000000u : 0x80008000u) : 0u;
    p.counters = a->counters;
    p.splits = 1;
    p.split_len = a->N;
    const bool count = a->counters != nullptr;
    const bool bf = a->dtype == FA_DTYPE_BF16, d64 = a->d == 64;
    const int c = a->causal, o32 = a->out_dtype;

    switch (plan.kind) {
    case kSweep:
        switch (plan.tq * 1000 + plan.tk) {
        case 256064: return fa::launch16_bf16_d128_c0(p, 0, count, a->stream);
        case 64032: return fa::launch16t_q64_k32(p, count, a->stream);
        case 64064: return fa::launch16t_q64_k64(p, count, a->stream);
        case 64128: return fa::launch16t_q64_k128(p, count, a->stream);
        case 128032: return fa::launch16t_q128_k32(p, count, a->stream);
        case 128064: return fa::launch16t_q128_k64(p, count, a->stream);
        case 128128: return fa::launch16t_q128_k128(p, count, a->stream);
        case 256032: return fa::launch16t_q256_k32(p, count, a->stream);
        case 256128: return fa::launch16t_q256_k128(p, count, a->stream);
        default: return FA_ERR_UNSUPPORTED;
        }
    case kPersistent:
        return bf ? fa::launch16p_bf16_d128(p, plan.grid, count, a->stream)
                  : fa::launch16p_f16_d128(p, plan.grid, count, a->stream);
    case kPersistentCausalWide:
        return bf ? fa::launch16pcw_bf16_d128(p, plan.grid, count, a->stream)
                  : fa::launch16pcw_f16_d128(p, plan.grid, count, a->stream);
    case kPerTile16:
        if (bf) {
            if (d64) return c ? fa::launch16_bf16_d64_c1(p, o32, count, a->stream)
                              : fa::launch16_bf16_d64_c0(p, o32, count, a->stream);
            return c ? fa::launch16_bf16_d128_c1(p, o32, count, a->stream)
                     : fa::launch16_bf16_d128_c0(p, o32, count, a->stream);
        }
        if (d64) return c ? fa::launch16_f16_d64_c1(p, o32, count, a->stream)
                          : fa::launch16_f16_d64_c0(p, o32, count, a->stream);
        return c ? fa::launch16_f16_d128_c1(p, o32, count, a->stream)
                 : fa::launch16_f16_d128_c0(p, o32, count, a->stream);
    case kPerTile32:
        return c ? fa::launch32_c1(p, a->d, count, a->stream) : fa::launch32_c0(p, a->d, count, a->stream);
    }
    return FA_ERR_UNSUPPORTED;
}

// The tile of the kernel a launch with these arguments runs.
int launch_tile(const fa_fwd_args* a, int* tile_q, int* tile_k) {
    if (!tile_q || !tile_k) return FA_ERR_INVALID;
    int st = check_args(a);
    if (st != FA_OK) return st;
    int cus = 0;
    st = check_device(&cus);
    if (st != FA_OK) return st;
    const LaunchPlan plan = plan_launch(a, cus);
    *tile_q = plan.tq;
    *tile_k = plan.tk;
    return FA_OK;
}

// Split-KV forward: argument checks, then the partial and merge kernels.
int run_split(const fa_fwd_args* a, float* o_part, float* lse_part, int splits) {
    int st = check_args(a);
    if (st != FA_OK) return st;
    if (!o_part || !lse_part || splits < 1) return FA_ERR_INVALID;
    if (a->out_dtype || a->counters || a->tile_q || a->tile_k) return FA_ERR_UNSUPPORTED;
    const bool causal = a->causal != 0;
    const bool f32 = a->dtype == FA_DTYPE_F32;
    const int tq = f32 ? 64 : fa::tile_q16(causal, a->d), tk = 64;
    // ranges of whole key tiles; as many as asked for, at most one per key tile
    const int nk = (a->N + tk - 1) / tk;
    const int per = (nk + std::min(splits, nk) - 1) / std::min(splits, nk);   // key tiles per range
    const int used = (nk + per - 1) / per;
    const uint64_t heads = (uint64_t)a->B * a->H, tiles = heads * ((a->N + tq - 1) / tq);
    if (tiles * used >= (1ull << 31)) return FA_ERR_UNSUPPORTED;
    const uint64_t e = elem_size(a->dtype), elems = heads * a->N * a->d;
    const uint64_t part_b = (uint64_t)splits * elems * 4, lpart_b = (uint64_t)splits * heads * a->N * 4;
    const void* bufs[5] = {a->q, a->k, a->v, a->o, a->lse};
    const uint64_t bufb[5] = {elems * e, elems * e, elems * e, elems * e, heads * a->N * 4};
    for (int i = 0; i < 5; ++i)
        if (overlaps(o_part, part_b, bufs[i], bufb[i]) || overlaps(lse_part, lpart_b, bufs[i], bufb[i]))
            return FA_ERR_INVALID;
    if (overlaps(o_part, part_b, lse_part, lpart_b)) return FA_ERR_INVALID;
    int cus = 0;
    st = check_device(&cus);
    if (st != FA_OK) return st;
    FwdParams p;
    p.q = a->q;
    p.k = a->k;
    p.v = a->v;
    p.o = o_part;
    p.lse = lse_part;
    p.N = a->N;
    p.tiles_q = (a->N + tq - 1) / tq;
    p.heads = (int)heads;
    p.total = (int)tiles;
    p.group = 1;
    p.c = std::fmax(std::fabs(a->scale) * 1.4426950408889634f, FLT_MIN);
    p.qsign = a->scale < 0.f ? (f32 ? 0x80000000u : 0x80008000u) : 0u;
    p.counters = nullptr;
    p.splits = used;
    p.split_len = per * tk;
    const bool bf = a->dtype == FA_DTYPE_BF16, d64 = a->d == 64;
    if (f32)
        return causal ? fa::launch32s_c1(p, a->d, a->o, a->lse, a->stream)
                      : fa::launch32s_c0(p, a->d, a->o, a->lse, a->stream);
    if (causal)
        return bf ? (d64 ? fa::launch16s_bf16_d64_c1(p, a->o, a->lse, a->stream)
                         : fa::launch16s_bf16_d128_c1(p, a->o, a->lse, a->stream))
                  : (d64 ? fa::launch16s_f16_d64_c1(p, a->o, a->lse, a->stream)
                         : fa::launch16s_f16_d128_c1(p, a->o, a->lse, a->stream));
    return bf ? (d64 ? fa::launch16s_bf16_d64_c0(p, a->o, a->lse, a->stream)
                     : fa::launch16s_bf16_d128_c0(p, a->o, a->lse, a->stream))
              : (d64 ? fa::launch16s_f16_d64_c0(p, a->o, a->lse, a->stream)
                     : fa::launch16s_f16_d128_c0(p, a->o, a->lse, a->stream));
}

}  // namespace

// The current device's check, shared with the other host layers of the
// library (fa_fwd_launch.h): FA_OK on gfx950, FA_ERR_UNSUPPORTED otherwise.
int fa::device_check(int* cus) { return check_device(cus); }

namespace {

fa_fwd_args plain_args(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                       int N, int d, float scale, int causal, void* stream, int dtype) {
    fa_fwd_args a;
    std::memset(&a, 0, sizeof(a));
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.B = B; a.H = H; a.N = N; a.d = d;
    a.scale = scale; a.causal = causal; a.stream = stream; a.dtype = dtype;
    return a;
}

}  // namespace

extern "C" {

int fa_fwd_ex(const fa_fwd_args* args) { return run(args); }

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
           float scale, int causal, void* stream, int dtype) {
    const fa_fwd_args a = plain_args(q, k, v, o, lse, B, H, N, d, scale, causal, stream, dtype);
    return run(&a);
}

int fa_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                float scale, int causal, void* stream) {
    return fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, stream, FA_DTYPE_BF16);
}

int fa_fwd_f16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
               float scale, int causal, void* stream) {
    return fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, stream, FA_DTYPE_F16);
}

int fa_fwd_f32(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
               float scale, int causal, void* stream) {
    return fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, stream, FA_DTYPE_F32);
}

int fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, float* o_part, float* lse_part,
                 int B, int H, int N, int d, float scale, int causal, int splits, void* stream, int dtype) {
    const fa_fwd_args a = plain_args(q, k, v, o, lse, B, H, N, d, scale, causal, stream, dtype);
    return run_split(&a, o_part, lse_part, splits);
}

int fa_fwd_launch_tile(const fa_fwd_args* args, int* tile_q, int* tile_k) { return launch_tile(args, tile_q, tile_k); }

int fa_fwd_split_count(int B, int H, int N, int d, int causal, int dtype, int* splits) {
    if (!splits || B <= 0 || H <= 0 || N <= 0 || (causal != 0 && causal != 1)) return FA_ERR_INVALID;
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    int cus = 0;
    const int st = check_device(&cus);
    if (st != FA_OK) return st;
    // the plain launch's work units: (head, query tile); without the mask
    // they cost the same, so ranges that bring them up to one per CU fill
    // the device; under the mask the longest unit costs twice the mean, so
    // units below twice the CU count leave the launch waiting on its longest
    // rows, and ranges cut them
    const int tq = dtype == FA_DTYPE_F32 ? 64 : fa::tile_q16(causal != 0, d);
    const uint64_t units = (uint64_t)B * H * ((uint64_t)(N + tq - 1) / tq);
    const uint64_t want = (causal ? 2ull * cus : (uint64_t)cus) / units;
    const uint64_t nk = ((uint64_t)N + 63) / 64;
    *splits = (int)std::max<uint64_t>(1, std::min<uint64_t>(std::min<uint64_t>(want, nk), 16));
    return FA_OK;
}

int fa_fwd_tile_shape(int dtype, int d, int causal, int* tile_q, int* tile_k) {
    if (!tile_q || !tile_k || (causal != 0 && causal != 1)) return FA_ERR_INVALID;
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    tile_shape(dtype, d, causal, tile_q, tile_k);
    return FA_OK;
}

const char* fa_strerror(int status) {
    switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported configuration";
    case FA_ERR_HIP: return "HIP runtime error";
    case FA_ERR_SCRATCH: return "problem exceeds the fixed scratch array of a no-allocation entry point";
    default: return "unknown status";
    }
}

const char* fa_build_info(void) {
    return "fa_fwd: offload-arch gfx950; flags: " FA_BUILD_FLAGS
           "; kernels: bf16/f16 d64 and d128 (d128: 256x64 tiles non-causal, 128x64 causal; d64: 128x64 tiles, "
           "three workgroups per CU; 32 query rows per wave; d128 persistent across query tiles, causal in pairs "
           "of 256-row tiles), causal on/off, "
           "out 16-bit/fp32, counters on/off; f32 d64/d128 (64x64 tiles), causal on/off, counters on/off; "
           "split-KV bf16/f16/f32 d64/d128 causal on/off (fp32 partials + merge); "
           "backward bf16/f16 d64/d128 causal on/off (dQ kernel, dK/dV kernel); "
           "standard materialising forward bf16/f16 d64/d128 (scores, softmax, output)";
}

}  // extern "C"
