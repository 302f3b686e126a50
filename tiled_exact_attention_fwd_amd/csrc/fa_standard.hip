// Standard attention forward (the baseline of "FlashAttention分块计算优化
// Transformer显存效率" §1.1 / §2.1): S and P materialised in HBM by three
// plain kernels.  16-bit inputs, d = 64 or 128.
//
//   scores   one workgroup = 32 query rows of one head, four waves taking
//            32-key blocks in turn; S^T = K Q^T on the matrix cores (fp32
//            accumulate), the K rows read in the permuted order of the tiled
//            kernel so that a lane's register octets hold 8 consecutive keys
//            of its query row; S = scale * QK^T rounded to the input type.
//   softmax  one wave per row: maximum, sum of exp, P = exp(S - m) / l
//            rounded to the input type (0 above the diagonal when causal),
//            LSE = m + ln l.  Rows of up to 8192 keys (a multiple of 8) are
//            read once into registers, 16 bytes per lane at a time; others
//            are read once per pass.
//   output   one workgroup = 32 query rows of one head, one wave per 32
//            output columns; O = P V on the matrix cores, P read as rows, V
//            gathered column-wise.
// The query blocks of one head run on one XCD (the workgroup renumbering of
// the tiled kernel), so that the head's K and V are re-read from one L2.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "fa_fwd.h"
#include "fa_fwd_launch.h"
#include "fa_fwd_kernels.h"
#include "fa_standard.h"

namespace fa {
namespace standard {

template <class T> __device__ __forceinline__ float to_f32(uint16_t h);
template <> __device__ __forceinline__ float to_f32<BF16>(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
template <> __device__ __forceinline__ float to_f32<F16>(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}
template <class T> __device__ __forceinline__ uint16_t to_bits(float x) { return (uint16_t)(pack2<T>(x, 0.f) & 0xffffu); }

__device__ __forceinline__ float wave_max(float x) {
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

template <class T, int D>
__global__ void __launch_bounds__(256) scores_kernel(const uint16_t* q, const uint16_t* k, uint16_t* s, int N,
                                                     float scale, int nqb) {
    constexpr int NS = D / 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 31, lh = lane >> 5;
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int hh = L / nqb, q0 = (L - hh * nqb) * 32;
    const size_t head = (size_t)hh * N * D;
    const uint32_t head_bytes = (uint32_t)N * D * 2;
    const auto rq = make_rsrc(q + head, head_bytes), rk = make_rsrc(k + head, head_bytes);
    u32x4_t qreg[NS];
#pragma unroll
    for (int st = 0; st < NS; ++st) qreg[st] = buf_load16(rq, (uint32_t)((q0 + li) * D + 16 * st + 8 * lh) * 2);
    const int prow = Fwd16<T, D, false, false, false>::perm_row(li);
    const bool vec = N % 8 == 0;
    uint16_t* const srow = s + ((size_t)hh * N + q0 + li) * N;
    for (int kb = wave * 32; kb < N; kb += 4 * 32) {
        f32x16_t acc = {};
#pragma unroll
        for (int st = 0; st < NS; ++st)
            acc = mma<T>(buf_load16(rk, (uint32_t)((kb + prow) * D + 16 * st + 8 * lh) * 2), qreg[st], acc);
        if (q0 + li >= N) continue;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            // registers 8 h2 .. 8 h2 + 7 hold keys kb + 16 h2 + 8 lh + 0..7
            const int key = kb + 16 * h2 + 8 * lh;
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = pack2<T>(acc[8 * h2 + 2 * i] * scale, acc[8 * h2 + 2 * i + 1] * scale);
            if (vec && key + 8 <= N) {
                *(u32x4_t*)(srow + key) = u32x4_t{w[0], w[1], w[2], w[3]};
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (key + e < N) srow[key + e] = (uint16_t)(w[e / 2] >> (16 * (e % 2)));
            }
        }
    }
}

template <class T>
__global__ void __launch_bounds__(256) softmax_kernel(const uint16_t* s, uint16_t* p, float* lse, int N, int causal,
                                                      int nrb) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int hh = blockIdx.x / nrb, row = (blockIdx.x - hh * nrb) * 4 + wave;
    if (row >= N) return;   // the whole wave; the kernel has no barrier
    const size_t off = ((size_t)hh * N + row) * N;
    const uint16_t* srow = s + off;
    uint16_t* prow = p + off;
    const int vis = causal ? row + 1 : N;   // keys the row sees
    float m = -INFINITY;
    for (int j = lane; j < vis; j += 64) m = fmaxf(m, to_f32<T>(srow[j]));
    m = wave_max(m);
    float l = 0.f;
    for (int j = lane; j < vis; j += 64) l += expf(to_f32<T>(srow[j]) - m);
    l = wave_sum(l);
    const float inv = 1.0f / l;
    for (int j = lane; j < N; j += 64) prow[j] = j < vis ? to_bits<T>(expf(to_f32<T>(srow[j]) - m) * inv) : (uint16_t)0;
    if (lane == 0) lse[(size_t)hh * N + row] = m + logf(l);
}

// One pass over a row held in registers: CH 16-byte chunks per lane
// (N % 8 == 0, N <= 512 CH).
template <class T, int CH>
__global__ void __launch_bounds__(256) softmax_row_kernel(const uint16_t* s, uint16_t* p, float* lse, int N,
                                                          int causal, int nrb) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int hh = blockIdx.x / nrb, row = (blockIdx.x - hh * nrb) * 4 + wave;
    if (row >= N) return;   // the whole wave; the kernel has no barrier
    const size_t off = ((size_t)hh * N + row) * N;
    const int vis = causal ? row + 1 : N;
    float x[CH][8];
    float m = -INFINITY;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int j0 = (c * 64 + lane) * 8;
        u32x4_t w = {0, 0, 0, 0};
        if (j0 < N) w = *(const u32x4_t*)(s + off + j0);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint16_t h = (uint16_t)(w[e / 2] >> (16 * (e % 2)));
            x[c][e] = j0 + e < vis ? to_f32<T>(h) : -INFINITY;
            m = fmaxf(m, x[c][e]);
        }
    }
    m = wave_max(m);
    float l = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            x[c][e] = expf(x[c][e] - m);
            l += x[c][e];
        }
    l = wave_sum(l);
    const float inv = 1.0f / l;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int j0 = (c * 64 + lane) * 8;
        if (j0 < N) {
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = pack2<T>(x[c][2 * i] * inv, x[c][2 * i + 1] * inv);
            *(u32x4_t*)(p + off + j0) = u32x4_t{w[0], w[1], w[2], w[3]};
        }
    }
    if (lane == 0) lse[(size_t)hh * N + row] = m + logf(l);
}

template <class T, int D>
__global__ void __launch_bounds__(64 * (D / 32)) output_kernel(const uint16_t* p, const uint16_t* v, uint16_t* o,
                                                               int N, int nqb) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 31, lh = lane >> 5;
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int hh = L / nqb, q0 = (L - hh * nqb) * 32, c0 = wave * 32;
    const uint16_t* prow = p + ((size_t)hh * N + q0 + li) * N;
    const uint16_t* vh = v + (size_t)hh * N * D;
    const bool rowok = q0 + li < N, vec = N % 8 == 0;
    f32x16_t acc = {};
    for (int kb = 0; kb < N; kb += 16) {
        // A: P[q0 + li][kb + 8 lh .. +7];  B: V[kb + 8 lh .. +7][c0 + li]
        const int col = kb + 8 * lh;
        u32x4_t a;
        if (rowok && vec && col + 8 <= N) {
            a = *(const u32x4_t*)(prow + col);
        } else {
            uint16_t e[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) e[i] = rowok && col + i < N ? prow[col + i] : (uint16_t)0;
            a = u32x4_t{e[0] | (uint32_t)e[1] << 16, e[2] | (uint32_t)e[3] << 16, e[4] | (uint32_t)e[5] << 16,
                        e[6] | (uint32_t)e[7] << 16};
        }
        uint16_t g[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) g[i] = col + i < N ? vh[(size_t)(col + i) * D + c0 + li] : (uint16_t)0;
        const u32x4_t b{g[0] | (uint32_t)g[1] << 16, g[2] | (uint32_t)g[3] << 16, g[4] | (uint32_t)g[5] << 16,
                        g[6] | (uint32_t)g[7] << 16};
        acc = mma<T>(a, b, acc);
    }
    // C[m][n]: lane (li, lh) holds column n = li, rows m = 8 (r / 4) + 4 lh + r % 4
    uint16_t* const oh = o + (size_t)hh * N * D;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = q0 + 8 * (r / 4) + 4 * lh + r % 4;
        if (row < N) oh[(size_t)row * D + c0 + li] = to_bits<T>(acc[r]);
    }
}

template <class T, int D>
int launch(const void* q, const void* k, const void* v, void* o, float* lse, void* s, void* p, int heads, int N,
           float scale, int causal, hipStream_t stream) {
    const int nqb = (N + 31) / 32, nrb = (N + 3) / 4;
    hipLaunchKernelGGL((scores_kernel<T, D>), dim3(nqb * heads), dim3(256), 0, stream, (const uint16_t*)q,
                       (const uint16_t*)k, (uint16_t*)s, N, scale, nqb);
    const dim3 sg(nrb * heads), sb(256);
    const uint16_t* sc = (const uint16_t*)s;
    uint16_t* pc = (uint16_t*)p;
    if (N % 8 == 0 && N <= 512 * 2)
        hipLaunchKernelGGL((softmax_row_kernel<T, 2>), sg, sb, 0, stream, sc, pc, lse, N, causal, nrb);
    else if (N % 8 == 0 && N <= 512 * 8)
        hipLaunchKernelGGL((softmax_row_kernel<T, 8>), sg, sb, 0, stream, sc, pc, lse, N, causal, nrb);
    else if (N % 8 == 0 && N <= 512 * 16)
        hipLaunchKernelGGL((softmax_row_kernel<T, 16>), sg, sb, 0, stream, sc, pc, lse, N, causal, nrb);
    else
        hipLaunchKernelGGL((softmax_kernel<T>), sg, sb, 0, stream, sc, pc, lse, N, causal, nrb);
    hipLaunchKernelGGL((output_kernel<T, D>), dim3(nqb * heads), dim3(64 * (D / 32)), 0, stream,
                       (const uint16_t*)p, (const uint16_t*)v, (uint16_t*)o, N, nqb);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace standard
}  // namespace fa

extern "C" int fa_standard_fwd(const void* q, const void* k, const void* v, void* o, float* lse, void* s, void* p,
                               int B, int H, int N, int d, float scale, int causal, void* stream, int dtype) {
    if (!q || !k || !v || !o || !lse || !s || !p) return FA_ERR_INVALID;
    if (((uintptr_t)s | (uintptr_t)p) & 15) return FA_ERR_INVALID;   // S / P rows are stored and read 16 B at a time
    if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return FA_ERR_INVALID;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID;
    if (!std::isfinite(scale)) return FA_ERR_INVALID;
    if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16) return FA_ERR_UNSUPPORTED;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    // (room for the 32-bit row offsets of a padded last block, as in the forward)
    if ((uint64_t)N * d * 4 >= (1ull << 31)) return FA_ERR_UNSUPPORTED;
    const uint64_t blocks = (uint64_t)B * H * ((N + 3) / 4);
    if (blocks >= (1ull << 31)) return FA_ERR_UNSUPPORTED;
    int cus = 0;
    const int dev_st = fa::device_check(&cus);
    if (dev_st != FA_OK) return dev_st;
    const int heads = B * H;
    const hipStream_t st = (hipStream_t)stream;
    if (dtype == FA_DTYPE_BF16)
        return d == 64 ? fa::standard::launch<fa::BF16, 64>(q, k, v, o, lse, s, p, heads, N, scale, causal, st)
                       : fa::standard::launch<fa::BF16, 128>(q, k, v, o, lse, s, p, heads, N, scale, causal, st);
    return d == 64 ? fa::standard::launch<fa::F16, 64>(q, k, v, o, lse, s, p, heads, N, scale, causal, st)
                   : fa::standard::launch<fa::F16, 128>(q, k, v, o, lse, s, p, heads, N, scale, causal, st);
}
