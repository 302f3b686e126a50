// Host layer of the attention backward (include/fa_bwd.h): argument checks,
// then the two kernels of fa_bwd_kernels.h on the caller's stream.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "fa_bwd.h"
#include "fa_bwd32_kernels.h"
#include "fa_bwd_kernels.h"
#include "fa_bwd_launch.h"
#include "fa_fwd.h"
#include "fa_fwd_launch.h"

// Work memory of fa_bwd_noalloc: the D array (one fp32 per query row of the
// launch), for callers that cannot allocate.  Every device the library runs
// on holds its own copy until the process ends.  In host code the name is a
// stand-in, not a device address: the address of the current device's copy
// comes from hipGetSymbolAddress, once per device, and only that address is
// handed to kernels.
static __device__ __align__(256) float scratch[FA_BWD_NOALLOC_MAX_ROWS];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
std::atomic<float*> g_scratch[kMaxDevices];   // device address of each device's copy

// The current device's copy of `scratch`, resolved on the first call made
// with that device current.
int scratch_for_current_device(float** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
    float* ptr = g_scratch[dev].load(std::memory_order_acquire);
    if (!ptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        ptr = g_scratch[dev].load(std::memory_order_relaxed);
        if (!ptr) {
            void* addr = nullptr;
            if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return FA_ERR_HIP;
            ptr = (float*)addr;
            g_scratch[dev].store(ptr, std::memory_order_release);
        }
    }
    *out = ptr;
    return FA_OK;
}

bool overlaps(const void* a, uint64_t an, const void* b, uint64_t bn) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bn && b0 < a0 + an;
}

int run(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout, void* dq,
        void* dk, void* dv, float* delta, int B, int H, int N, int d, float scale, int causal, void* stream,
        int dtype, bool noalloc = false, bool o32 = false) {
    // noalloc: delta is ignored and the D array lives in `scratch`;
    // o32: o is fp32 whatever the element type
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || (!noalloc && !delta)) return FA_ERR_INVALID;
    if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return FA_ERR_INVALID;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID;
    if (!std::isfinite(scale)) return FA_ERR_INVALID;
    if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_F32) return FA_ERR_UNSUPPORTED;
    const uint64_t e = dtype == FA_DTYPE_F32 ? 4 : 2;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    // per-head bytes, with room for the 32-bit row offsets of the padded
    // last block (rows up to N + 255) as in the forward
    if ((uint64_t)N * d * 4 >= (1ull << 31)) return FA_ERR_UNSUPPORTED;
    const uint64_t heads = (uint64_t)B * H, nblk = ((uint64_t)N + 127) / 128;
    if (heads * nblk >= (1ull << 31)) return FA_ERR_UNSUPPORTED;
    const uint64_t tb = heads * N * d * e, sb = heads * N * 4, ob = o32 ? heads * N * d * 4 : tb;
    const void* ins[6] = {q, k, v, o, dout, lse};
    const uint64_t inb[6] = {tb, tb, tb, ob, tb, sb};
    void* outs[4] = {dq, dk, dv, delta};
    const uint64_t outb[4] = {tb, tb, tb, sb};
    const int nouts = noalloc ? 3 : 4;
    for (int i = 0; i < nouts; ++i) {
        for (int j = 0; j < 6; ++j)
            if (overlaps(outs[i], outb[i], ins[j], inb[j])) return FA_ERR_INVALID;
        for (int j = i + 1; j < nouts; ++j)
            if (overlaps(outs[i], outb[i], outs[j], outb[j])) return FA_ERR_INVALID;
    }
    if (noalloc && heads * N > (uint64_t)FA_BWD_NOALLOC_MAX_ROWS) return FA_ERR_SCRATCH;
    int cus = 0;
    const int dev_st = fa::device_check(&cus);
    if (dev_st != FA_OK) return dev_st;
    if (noalloc) {
        const int sst = scratch_for_current_device(&delta);
        if (sst != FA_OK) return sst;
    }
    if (dtype == FA_DTYPE_F32) {
        fa::bwd::BwdParams32 p32;
        p32.q = (const float*)q; p32.k = (const float*)k; p32.v = (const float*)v;
        p32.o = (const float*)o; p32.dout = (const float*)dout; p32.lse = lse;
        p32.dq = (float*)dq; p32.dk = (float*)dk; p32.dv = (float*)dv; p32.delta = delta;
        p32.N = N;
        p32.nblk = (int)nblk;
        p32.c = scale * fa::bwd::kLog2e;
        p32.scale = scale;
        return fa::bwd::launch_bwd_f32(p32, (int)heads, d, causal != 0, stream) == 0 ? FA_OK : FA_ERR_HIP;
    }
    fa::bwd::BwdParams p;
    p.q = (const uint16_t*)q; p.k = (const uint16_t*)k; p.v = (const uint16_t*)v;
    p.o = o32 ? nullptr : (const uint16_t*)o; p.o32 = o32 ? (const float*)o : nullptr;
    p.dout = (const uint16_t*)dout; p.lse = lse;
    p.dq = (uint16_t*)dq; p.dk = (uint16_t*)dk; p.dv = (uint16_t*)dv; p.delta = delta;
    p.N = N;
    p.heads = (int)heads;
    p.nblk = (int)nblk;
    p.c = scale * fa::bwd::kLog2e;
    p.scale = scale;
    const bool c = causal != 0;
    int rc;
    if (dtype == FA_DTYPE_BF16)
        rc = d == 64 ? fa::bwd::launch_bwd_bf16_d64(p, (int)heads, cus, c, stream)
                     : fa::bwd::launch_bwd_bf16_d128(p, (int)heads, cus, c, stream);
    else
        rc = d == 64 ? fa::bwd::launch_bwd_f16_d64(p, (int)heads, cus, c, stream)
                     : fa::bwd::launch_bwd_f16_d128(p, (int)heads, cus, c, stream);
    return rc == 0 ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout, void* dq,
           void* dk, void* dv, float* delta, int B, int H, int N, int d, float scale, int causal, void* stream,
           int dtype) {
    return run(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, scale, causal, stream, dtype);
}

int fa_bwd_o32(const void* q, const void* k, const void* v, const float* o, const float* lse, const void* dout,
               void* dq, void* dk, void* dv, float* delta, int B, int H, int N, int d, float scale, int causal,
               void* stream, int dtype) {
    return run(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, scale, causal, stream, dtype, false, true);
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                   void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, void* stream,
                   int dtype) {
    return run(q, k, v, o, lse, dout, dq, dk, dv, nullptr, B, H, N, d, scale, causal, stream, dtype, true);
}

int fa_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                void* dq, void* dk, void* dv, float* delta, int B, int H, int N, int d, float scale, int causal,
                void* stream) {
    return run(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, scale, causal, stream, FA_DTYPE_BF16);
}

int fa_bwd_f16(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
               void* dq, void* dk, void* dv, float* delta, int B, int H, int N, int d, float scale, int causal,
               void* stream) {
    return run(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, scale, causal, stream, FA_DTYPE_F16);
}

int fa_bwd_f32(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
               void* dq, void* dk, void* dv, float* delta, int B, int H, int N, int d, float scale, int causal,
               void* stream) {
    return run(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, scale, causal, stream, FA_DTYPE_F32);
}

}  // extern "C"
