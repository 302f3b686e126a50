// fp32 attention backward for gfx950: the same two kernels and the same
// arithmetic as fa_bwd_kernels.h (P rebuilt from the forward's log-sum-exp,
// D = rowsum(dO * O), dS = P (dP - D), dQ = scale dS K, dK = scale dS^T Q,
// dV = P^T dO) on the fp32 matrix cores, v_mfma_f32_32x32x2_f32.
//
// Layout of that instruction (C = A B, 2-deep steps): lane (li, lh)
// supplies A[li][lh] and B[lh][li] and holds C[8 (r / 4) + 4 lh + r % 4][li]
// in register r.  The product of a 32 x 32 result block with a third matrix
// takes step t = 0..15 with lane half lh's k index standing for row
// 8 (t / 4) + 4 lh + t % 4 of the block -- register t of that lane -- so the
// B operand is the register itself and the A operand one fp32 read from LDS
// at that row.  Nothing is rounded below fp32.  Tiles pass through LDS
// single-buffered (64 rows, padded pitch); this path serves small fp32
// problems, where the launch dominates.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_bwd_kernels.h"

namespace fa {
namespace bwd {

struct BwdParams32 {
    const float *q, *k, *v, *o, *dout;
    const float* lse;
    float *dq, *dk, *dv;
    float* delta;
    int N;
    int nblk;      // 128-row blocks per head
    float c;       // scale * log2(e)
    float scale;
};

template <int D>
struct Geo32 {
    static constexpr int NS = D / 2;             // 2-deep steps over the head dimension
    static constexpr int NDB = D / 32;
    static constexpr int PITCH = D * 4 + 16;     // LDS row pitch in bytes
    static constexpr int TILE = 64;
    static constexpr int CHUNKS = TILE * D / 4;  // 16-byte pieces per tile
};

__device__ __forceinline__ f32x16_t mma32(float a, float b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// rows [r0, r0 + 64) of one head into LDS; rows past the head read as zeros
template <int D>
__device__ __forceinline__ void load_tile32(__amdgpu_buffer_rsrc_t r, uint8_t* lds, int r0, int tid) {
    using G = Geo32<D>;
#pragma unroll
    for (int i = tid; i < G::CHUNKS; i += 256) {
        const int row = i / (D / 4), ch = i % (D / 4);
        *(u32x4_t*)(lds + row * G::PITCH + ch * 16) = buf_load16(r, (uint32_t)(((r0 + row) * D + ch * 4) * 4));
    }
}

template <int D>
__device__ __forceinline__ float lds_at(const uint8_t* lds, int row, int col) {
    return *(const float*)(lds + row * Geo32<D>::PITCH + col * 4);
}

// one row's B operands: lane (li, lh) gets row[2 s + lh] for every step s
template <int D>
__device__ __forceinline__ void load_row_operands(__amdgpu_buffer_rsrc_t r, int row, int lh, float* x) {
#pragma unroll
    for (int s4 = 0; s4 < D / 8; ++s4) {
        const u32x4_t lo = buf_load16(r, (uint32_t)((row * D + 8 * s4) * 4));
        const u32x4_t hi = buf_load16(r, (uint32_t)((row * D + 8 * s4 + 4) * 4));
        x[4 * s4 + 0] = __uint_as_float(lh ? lo[1] : lo[0]);
        x[4 * s4 + 1] = __uint_as_float(lh ? lo[3] : lo[2]);
        x[4 * s4 + 2] = __uint_as_float(lh ? hi[1] : hi[0]);
        x[4 * s4 + 3] = __uint_as_float(lh ? hi[3] : hi[2]);
    }
}

// a 32 x D transposed accumulator (register r of acc[db] = column
// 32 db + 8 (r / 4) + 4 lh + r % 4 of row `row`) times mul, as fp32
template <int D>
__device__ __forceinline__ void store_rows32(float* out, int row, int N, const f32x16_t* acc, float mul, int lh) {
    if (row >= N) return;
    float* p = out + (size_t)row * D + 4 * lh;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            *(__attribute__((address_space(1))) f32x4_t*)(p + 32 * db + 8 * g) =
                f32x4_t{acc[db][4 * g] * mul, acc[db][4 * g + 1] * mul, acc[db][4 * g + 2] * mul,
                        acc[db][4 * g + 3] * mul};
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256) dq_kernel32(BwdParams32 p) {
    using G = Geo32<D>;
    __shared__ __attribute__((aligned(16))) uint8_t ks[G::TILE * G::PITCH];
    __shared__ __attribute__((aligned(16))) uint8_t vs[G::TILE * G::PITCH];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 31, lh = lane >> 5;
    const int N = p.N;
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int hh = L / p.nblk;
    int qb = L - hh * p.nblk;
    if (CAUSAL) qb = p.nblk - 1 - qb;
    const int q0 = qb * 128, qw = q0 + 32 * wave, q = qw + li;
    const size_t head = (size_t)hh * N * D;
    const uint32_t hb = (uint32_t)N * D * 4;
    const auto rq = make_rsrc(p.q + head, hb), rk = make_rsrc(p.k + head, hb), rv = make_rsrc(p.v + head, hb);
    const auto ro = make_rsrc(p.o + head, hb), rdo = make_rsrc(p.dout + head, hb);

    float qreg[G::NS], dreg[G::NS], oreg[G::NS];
    load_row_operands<D>(rq, q, lh, qreg);
    load_row_operands<D>(rdo, q, lh, dreg);
    load_row_operands<D>(ro, q, lh, oreg);
    float dsum = 0.f;
#pragma unroll
    for (int s = 0; s < G::NS; ++s) dsum += dreg[s] * oreg[s];
    dsum = sum_halves(dsum);
    const bool qok = q < N;
    if (qok && lh == 0) p.delta[(size_t)hh * N + q] = dsum;
    const float lse2 = qok ? p.lse[(size_t)hh * N + q] * kLog2e : __builtin_inff();
    const float c = p.c;

    f32x16_t acc[G::NDB];
#pragma unroll
    for (int db = 0; db < G::NDB; ++db) acc[db] = f32x16_t{};
    const int kend = CAUSAL ? min(N, q0 + 128) : N;
    const int nkt = (kend + G::TILE - 1) / G::TILE;
    for (int kt = 0; kt < nkt; ++kt) {
        __syncthreads();
        load_tile32<D>(rk, ks, kt * G::TILE, tid);
        load_tile32<D>(rv, vs, kt * G::TILE, tid);
        __syncthreads();
        for (int sub = 0; sub < 2; ++sub) {
            const int k0 = kt * G::TILE + 32 * sub;
            if (k0 >= N || (CAUSAL && k0 > qw + 31)) continue;   // wave-uniform
            f32x16_t st{}, dpt{};
#pragma unroll
            for (int s = 0; s < G::NS; ++s) {
                st = mma32(lds_at<D>(ks, 32 * sub + li, 2 * s + lh), qreg[s], st);
                dpt = mma32(lds_at<D>(vs, 32 * sub + li, 2 * s + lh), dreg[s], dpt);
            }
            float ds[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = k0 + 8 * (r / 4) + 4 * lh + (r % 4);
                const bool vis = key < N && (!CAUSAL || key <= q);
                ds[r] = vis ? __builtin_amdgcn_exp2f(c * st[r] - lse2) * (dpt[r] - dsum) : 0.f;
            }
            // dQ^T += K^T dS^T
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const int kl = 32 * sub + 8 * (t / 4) + 4 * lh + (t % 4);
#pragma unroll
                for (int db = 0; db < G::NDB; ++db) acc[db] = mma32(lds_at<D>(ks, kl, 32 * db + li), ds[t], acc[db]);
            }
        }
    }
    store_rows32<D>(p.dq + head, q, N, acc, p.scale, lh);
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256) dkdv_kernel32(BwdParams32 p) {
    using G = Geo32<D>;
    __shared__ __attribute__((aligned(16))) uint8_t qs[G::TILE * G::PITCH];
    __shared__ __attribute__((aligned(16))) uint8_t dos[G::TILE * G::PITCH];
    __shared__ __attribute__((aligned(16))) float lses[G::TILE];
    __shared__ __attribute__((aligned(16))) float dls[G::TILE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 31, lh = lane >> 5;
    const int N = p.N;
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int hh = L / p.nblk;
    const int kb = L - hh * p.nblk;
    const int k0 = kb * 128, kw = k0 + 32 * wave, key = kw + li;
    const size_t head = (size_t)hh * N * D;
    const uint32_t hb = (uint32_t)N * D * 4;
    const auto rq = make_rsrc(p.q + head, hb), rk = make_rsrc(p.k + head, hb), rv = make_rsrc(p.v + head, hb);
    const auto rdo = make_rsrc(p.dout + head, hb);
    const float* lse = p.lse + (size_t)hh * N;
    const float* delta = p.delta + (size_t)hh * N;

    float kreg[G::NS], vreg[G::NS];
    load_row_operands<D>(rk, key, lh, kreg);
    load_row_operands<D>(rv, key, lh, vreg);
    const float c = p.c;
    f32x16_t acck[G::NDB], accv[G::NDB];
#pragma unroll
    for (int db = 0; db < G::NDB; ++db) {
        acck[db] = f32x16_t{};
        accv[db] = f32x16_t{};
    }
    const int nqt = (N + G::TILE - 1) / G::TILE;
    const int qt0 = CAUSAL ? k0 / G::TILE : 0;
    for (int qt = qt0; qt < nqt; ++qt) {
        __syncthreads();
        load_tile32<D>(rq, qs, qt * G::TILE, tid);
        load_tile32<D>(rdo, dos, qt * G::TILE, tid);
        if (tid < G::TILE) {
            const int r = qt * G::TILE + tid;
            lses[tid] = r < N ? lse[r] * kLog2e : __builtin_inff();   // rows past N: P = 0
            dls[tid] = r < N ? delta[r] : 0.f;
        }
        __syncthreads();
        for (int sub = 0; sub < 2; ++sub) {
            const int qs0 = qt * G::TILE + 32 * sub;
            if (qs0 >= N || (CAUSAL && qs0 + 31 < kw)) continue;   // wave-uniform
            // S and dP: A = Q / dO rows (query qs0 + li), B = this wave's K / V rows
            f32x16_t st{}, dpt{};
#pragma unroll
            for (int s = 0; s < G::NS; ++s) {
                st = mma32(lds_at<D>(qs, 32 * sub + li, 2 * s + lh), kreg[s], st);
                dpt = mma32(lds_at<D>(dos, 32 * sub + li, 2 * s + lh), vreg[s], dpt);
            }
            float pr[16], ds[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ql = 32 * sub + 8 * (r / 4) + 4 * lh + (r % 4);
                const bool vis = !CAUSAL || key <= qt * G::TILE + ql;
                pr[r] = vis ? __builtin_amdgcn_exp2f(c * st[r] - lses[ql]) : 0.f;
                ds[r] = pr[r] * (dpt[r] - dls[ql]);
            }
            // dV^T += dO^T P,  dK^T += Q^T dS
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const int ql = 32 * sub + 8 * (t / 4) + 4 * lh + (t % 4);
#pragma unroll
                for (int db = 0; db < G::NDB; ++db) {
                    accv[db] = mma32(lds_at<D>(dos, ql, 32 * db + li), pr[t], accv[db]);
                    acck[db] = mma32(lds_at<D>(qs, ql, 32 * db + li), ds[t], acck[db]);
                }
            }
        }
    }
    store_rows32<D>(p.dk + head, key, N, acck, p.scale, lh);
    store_rows32<D>(p.dv + head, key, N, accv, 1.0f, lh);
}

}  // namespace bwd
}  // namespace fa
