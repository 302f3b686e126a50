// Probes of include/fa_probe.h: the clock probe (shader cycles counted over a
// fixed stretch of real time, by one wave on each of 64 CUs) and the
// issue-rate probe of the key loop's instruction mixes.

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

// ---------------------------------------------------------------------------
// Issue-rate probe (fa_issue_probe): the key loop's instruction mixes on
// register data, two waves per SIMD.  Every result stays live through the
// loop (register pins) and feeds the store at the end, so nothing is
// optimised away; the stores go to the caller's buffer only.
// ---------------------------------------------------------------------------
namespace {

typedef __bf16 probe_bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 probe_bf16x2_t __attribute__((ext_vector_type(2)));
typedef float probe_f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned probe_u32x4_t __attribute__((ext_vector_type(4)));

template <class X> __device__ __forceinline__ void keep(X& x) { asm volatile("" : "+v"(x)); }

// one softmax pair of the kernels on scores x[2i], x[2i+1]: x = c s - m
// (fma), 2^x (exp), pack to bf16, add both terms to a running sum
__device__ __forceinline__ void softmax_pair(float* x, unsigned* w, float* sum, int i) {
    float x0 = __builtin_fmaf(x[2 * i], 0.18f, -1.5f), x1 = __builtin_fmaf(x[2 * i + 1], 0.18f, -1.5f);
    keep(x0);
    keep(x1);
    x0 = __builtin_amdgcn_exp2f(x0);
    x1 = __builtin_amdgcn_exp2f(x1);
    keep(x0);
    keep(x1);
    const probe_bf16x2_t v = {(__bf16)x0, (__bf16)x1};
    w[i] ^= __builtin_bit_cast(unsigned, v);
    sum[i & 3] += x0;
    sum[i & 3] += x1;
    keep(w[i]);
    keep(sum[i & 3]);
    x[2 * i] = x0;
    x[2 * i + 1] = x1;
}

template <int MODE>
__global__ void __launch_bounds__(256) issue_probe_kernel(unsigned long long* out, int iters) {
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = 0.01f * (i + 1) + threadIdx.x * 1e-6f;
    float sum[4] = {0.f, 0.f, 0.f, 0.f};
    unsigned w[8] = {};
    probe_f32x16_t acc[4] = {};
    const probe_u32x4_t a = {0x3f803f80u ^ threadIdx.x, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
    const probe_u32x4_t b = {0x3f003f00u, 0x3f003f00u ^ threadIdx.x, 0x3f003f00u, 0x3f003f00u};
    __syncthreads();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it) {
        if constexpr (MODE == FA_PROBE_EXP) {
#pragma unroll
            for (int i = 0; i < 16; ++i) { x[i] = __builtin_amdgcn_exp2f(-x[i]); keep(x[i]); }
        } else if constexpr (MODE == FA_PROBE_FMA) {
#pragma unroll
            for (int i = 0; i < 16; ++i) { x[i] = __builtin_fmaf(x[i], 0.18f, -1.5f); keep(x[i]); }
        } else if constexpr (MODE == FA_PROBE_ADD) {
#pragma unroll
            for (int i = 0; i < 16; ++i) { x[i] = x[i] + 0.18f; keep(x[i]); }
        } else if constexpr (MODE == FA_PROBE_PACK) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const probe_bf16x2_t v = {(__bf16)x[2 * i], (__bf16)x[2 * i + 1]};
                w[i] ^= __builtin_bit_cast(unsigned, v);
                keep(w[i]);
            }
        } else if constexpr (MODE == FA_PROBE_SOFTMAX) {
#pragma unroll
            for (int i = 0; i < 4; ++i) softmax_pair(x, w, sum, i);
        } else {
            // MFMA, alone or with 1 (d = 64) or 1/2 (d = 128) softmax pair each
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                acc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(probe_bf16x8_t, a),
                                                                 __builtin_bit_cast(probe_bf16x8_t, b), acc[g], 0, 0, 0);
                if constexpr (MODE == FA_PROBE_MIX64) softmax_pair(x, w, sum, g);
                if constexpr (MODE == FA_PROBE_MIX128) {
                    if (g & 1) softmax_pair(x, w, sum, g >> 1);
                }
            }
        }
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    float sink = sum[0] + sum[1] + sum[2] + sum[3];
#pragma unroll
    for (int i = 0; i < 16; ++i) sink += x[i];
#pragma unroll
    for (int i = 0; i < 8; ++i) sink += (float)w[i];
#pragma unroll
    for (int g = 0; g < 4; ++g) sink += acc[g][0] + acc[g][15];
    if ((threadIdx.x & 63) == 0) {
        const size_t wv = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
        unsigned long long* o = (unsigned long long*)out + 3 * wv;
        *(__attribute__((address_space(1))) unsigned long long*)(o) = t1 - t0;
        // (the sink is never this value; the comparison keeps the work live)
        *(__attribute__((address_space(1))) unsigned long long*)(o + 1) = r0 + (sink == 12345.678f ? 1 : 0);
        *(__attribute__((address_space(1))) unsigned long long*)(o + 2) = r1;
    }
}

}  // namespace

extern "C" int fa_issue_probe(int mode, int iters, unsigned long long* out, long long out_len, void* stream) {
    if (!out || mode < 0 || mode >= FA_PROBE_MODES || iters < 1 || iters > FA_PROBE_MAX_ITERS) return FA_ERR_INVALID;
    int cus = 0;
    const int st = fa::device_check(&cus);
    if (st != FA_OK) return st;
    const int blocks = 2 * cus;                      // two four-wave workgroups per CU
    if (out_len < 3LL * 4 * blocks) return FA_ERR_INVALID;
    const hipStream_t s = (hipStream_t)stream;
    switch (mode) {
    case FA_PROBE_EXP: hipLaunchKernelGGL(issue_probe_kernel<FA_PROBE_EXP>, dim3(blocks), dim3(256), 0, s, out, iters); break;
    case FA_PROBE_FMA: hipLaunchKernelGGL(issue_probe_kernel<FA_PROBE_FMA>, dim3(blocks), dim3(256), 0, s, out, iters); break;
    case FA_PROBE_ADD: hipLaunchKernelGGL(issue_probe_kernel<FA_PROBE_ADD>, dim3(blocks), dim3(256), 0, s, out, iters); break;
    case FA_PROBE_PACK: hipLaunchKernelGGL(issue_probe_kernel<FA_PROBE_PACK>, dim3(blocks), dim3(256), 0, s, out, iters); break;
    case FA_PROBE_SOFTMAX:
        hipLaunchKernelGGL(issue_probe_kernel<FA_PROBE_SOFTMAX>, dim3(blocks), dim3(256), 0, s, out, iters);
        break;
    case FA_PROBE_MFMA: hipLaunchKernelGGL(issue_probe_kernel<FA_PROBE_MFMA>, dim3(blocks), dim3(256), 0, s, out, iters); break;
    case FA_PROBE_MIX64:
        hipLaunchKernelGGL(issue_probe_kernel<FA_PROBE_MIX64>, dim3(blocks), dim3(256), 0, s, out, iters);
        break;
    default:
        hipLaunchKernelGGL(issue_probe_kernel<FA_PROBE_MIX128>, dim3(blocks), dim3(256), 0, s, out, iters);
        break;
    }
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}
