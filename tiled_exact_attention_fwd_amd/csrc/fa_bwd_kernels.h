// Attention backward kernels for gfx950 (CDNA4, wave64, MFMA), with the
// probabilities recomputed tile by tile from the forward's log-sum-exp
// ("Flash Attention 原理", two pillars: recomputation).  The gradients are
// those of the forward of "FlashAttention分块计算优化Transformer显存效率"
// §1.1 / §2.2, O = softmax(scale Q K^T [causal]) V:
//
//   P = exp2(c s - LSE log2 e) with c = scale log2 e    (0 where masked)
//   D = rowsum(dO * O),  dS = P * (dO V^T - D)
//   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO
//
// Two kernels, launched in this order on one stream:
//
//   dq_kernel    one workgroup = 256 query rows of one head at d = 128 (8
//                waves x 32 rows; 128 rows and 4 waves at d = 64); the
//                wave's Q and dO rows stay in registers, K and V
//                tiles of 64 keys pass through LDS.  Per 32-key block it
//                computes S^T = K Q^T and dP^T = V dO^T (a lane holds one
//                query), dS^T, and dQ^T += K^T dS^T; it also computes D for
//                its rows from O and dO and writes it for the second kernel.
//   dkdv_kernel  one workgroup = 256 keys of one head at d = 128 (8 waves x
//                32 keys; 128 keys and 4 waves at d = 64); the wave's K rows
//                stay in registers, its V rows too at d = 64 and in LDS at
//                d = 128; Q and dO tiles of 64 queries (with their LSE and D)
//                pass through LDS.  Per
//                32-query block it computes S = Q K^T and dP = dO V^T (a lane
//                holds one key), dS, and dV^T += dO^T P, dK^T += Q^T dS.
//
// Each kernel recomputes S and dP for the pairs it visits, so the backward
// runs seven N x N x d products per head where one that stored partial dQ
// sums would run five; in exchange neither kernel needs atomics or a
// reduction buffer and the results are deterministic.  (A five-product
// kernel that adds each key block's share of dQ with float atomics measured
// 4% faster at 4096 rows, d = 128, and half again slower at d = 64, where a
// key block's dQ atomics meet half the matrix work.)
//
// MFMA layout (v_mfma_f32_32x32x16_{bf16,f16}, C = A B): lane (li, lh) of
// the wave (li = lane % 32, lh = lane / 32) supplies A[li][8 lh .. 8 lh + 7]
// and B[8 lh .. 8 lh + 7][li] of each 16-deep step, and holds
// C[8 (r / 4) + 4 lh + r % 4][li] in accumulator register r.  The product of
// a 32-row block of S (or S^T) with a third matrix takes registers 8t..8t+7
// of the first result as the B operand of step t: its k index e then stands
// for row 16 t + 4 lh + 8 (e / 4) + e % 4, and the A operand is read with
// the same index order from a row-major tile in LDS by the transposing read
// ds_read_b64_tr_b16 (each 16-lane group hands lane s four consecutive rows
// of column s of a 4 x 16 block whose row s / 4, columns 4 (s % 4) .. +3 it
// addressed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_fwd_kernels.h"

namespace fa {
namespace bwd {

constexpr float kLog2e = 1.44269504088896340736f;

struct BwdParams {
    const uint16_t *q, *k, *v, *o, *dout;
    const float* o32;  // O in fp32 (dq_kernel<.., O32 = true>; o unused then)
    const float* lse;
    uint16_t *dq, *dk, *dv;
    float* delta;
    int N;
    int heads;     // B * H
    int nblk;      // query blocks per head (dq_kernel, DqShape<D>::ROWS rows each)
    int nblk_k;    // key blocks per head (dkdv_kernel, DkdvShape<D>::KEYS keys each)
    int group;     // causal: heads per group of dq_kernel's block order
    int group_k;   // causal: heads per group of dkdv_kernel's block order
    float c;       // scale * log2(e)
    float scale;
};

template <class T> __device__ __forceinline__ float to_f32(uint32_t h);
template <> __device__ __forceinline__ float to_f32<BF16>(uint32_t h) { return __uint_as_float(h << 16); }
template <> __device__ __forceinline__ float to_f32<F16>(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// dot product of two 8-element 16-bit vectors in fp32
template <class T> __device__ __forceinline__ float dot8(u32x4_t a, u32x4_t b) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        s += to_f32<T>(a[i] & 0xffffu) * to_f32<T>(b[i] & 0xffffu);
        s += to_f32<T>(a[i] >> 16) * to_f32<T>(b[i] >> 16);
    }
    return s;
}

// the same with the second vector in fp32 (elements 0..3 in lo, 4..7 in hi),
// summed in the same order: equal bits when it holds the 16-bit values
template <class T> __device__ __forceinline__ float dot8f(u32x4_t a, u32x4_t lo, u32x4_t hi) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t b0 = i < 2 ? lo[2 * i] : hi[2 * i - 4], b1 = i < 2 ? lo[2 * i + 1] : hi[2 * i - 3];
        s += to_f32<T>(a[i] & 0xffffu) * __uint_as_float(b0);
        s += to_f32<T>(a[i] >> 16) * __uint_as_float(b1);
    }
    return s;
}

template <int D>
struct Geo {
    static constexpr int NS = D / 16;          // 16-deep steps over the head dimension
    static constexpr int NDB = D / 32;         // 32-column blocks of the head dimension
    static constexpr int PITCH = D * 2 + 16;   // LDS row pitch in bytes (padded against bank conflicts)
    static constexpr int TILE = 64;            // rows per LDS tile
    static constexpr int CHUNKS = TILE * D / 8;  // 16-byte pieces per tile
};

// A tile is rows [r0, r0 + 64) of one head (row-major, D columns, 16-bit),
// copied HBM -> registers -> LDS (row pitch Geo<D>::PITCH): the loads of the
// next tile are issued before the current tile is computed and stored to the
// other LDS buffer after it, so their latency is hidden.  Rows past the head's end read as zeros through the buffer
// resource's extent.
template <int D, int NT = 256>
struct TileRegs {
    static constexpr int PER = Geo<D>::CHUNKS / NT;    // 16-byte pieces per thread
    u32x4_t x[PER];
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int r0, int tid) {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int i = tid + NT * u, row = i / (D / 8), ch = i % (D / 8);
            x[u] = buf_load16(r, (uint32_t)(((r0 + row) * D + ch * 8) * 2));
        }
    }
    __device__ __forceinline__ void store(uint8_t* lds, int tid) const {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int i = tid + NT * u, row = i / (D / 8), ch = i % (D / 8);
            *(u32x4_t*)(lds + row * Geo<D>::PITCH + ch * 16) = x[u];
        }
    }
};

// A operand of step t taken from a row-major LDS tile: rows blk + 16 t + 4 lh
// + 8 (e / 4) + e % 4 (e = 0..7), column col0 + li (col0 a multiple of 32).
template <int D>
__device__ __forceinline__ u32x4_t tr_operand(const uint8_t* lds, int blk, int t, int col0, int lane) {
    using G = Geo<D>;
    const int s = lane & 15, grp = lane >> 4, lh = lane >> 5;
    const uint8_t* p = lds + (blk + 16 * t + 4 * lh + (s >> 2)) * G::PITCH + (col0 + 16 * (grp & 1) + 4 * (s & 3)) * 2;
    const u32x2_t a = lds_read_tr(p), b = lds_read_tr(p + 8 * G::PITCH);
    return u32x4_t{a[0], a[1], b[0], b[1]};
}

// Causal launches: workgroup -> (head, rank), where rank 0 is a head's most
// expensive block.  With a head count divisible by 8, XCD x (which runs
// workgroups b = x mod 8) owns heads x, x + 8, ... and takes them in groups
// of `group` heads, one group after the other, rank-major inside a group:
// the launch ends with the cheap blocks of the last group, and the K / V (or
// Q / dO) tiles re-read by a group's blocks stay in the XCD's L2 while the
// group runs.  The last group of an XCD may hold fewer heads.
__device__ __forceinline__ void causal_order(int bid, int heads, int nblk, int group, int& hh, int& rank) {
    if (heads % kNumXcd == 0) {
        const int x = bid % kNumXcd, s = bid / kNumXcd, hpx = heads / kNumXcd;
        const int gi = s / (group * nblk), r = s - gi * group * nblk;
        const int g = min(group, hpx - gi * group);
        rank = r / g;
        hh = (gi * group + r - rank * g) * kNumXcd + x;
    } else {
        rank = bid / heads;
        hh = bid - rank * heads;
    }
}

// 16 fp32 results -> the two B operands (registers 8t .. 8t + 7 each)
template <class T>
__device__ __forceinline__ void pack_b(const float* x, u32x4_t* b) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
        b[t] = u32x4_t{pack2<T>(x[8 * t + 0], x[8 * t + 1]), pack2<T>(x[8 * t + 2], x[8 * t + 3]),
                       pack2<T>(x[8 * t + 4], x[8 * t + 5]), pack2<T>(x[8 * t + 6], x[8 * t + 7])};
}

// Stores a 32 x D transposed accumulator (acc[db] register r = column
// 32 db + 8 (r / 4) + 4 lh + r % 4 of row `row`) times `mul` as 16-bit.
template <class T, int D>
__device__ __forceinline__ void store_rows(uint16_t* out, int row, int N, const f32x16_t* acc, float mul, int lh) {
    if (row >= N) return;
    uint16_t* p = out + (size_t)row * D + 4 * lh;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const u32x2_t w{pack2<T>(acc[db][4 * g] * mul, acc[db][4 * g + 1] * mul),
                            pack2<T>(acc[db][4 * g + 2] * mul, acc[db][4 * g + 3] * mul)};
            *(__attribute__((address_space(1))) u32x2_t*)(p + 32 * db + 8 * g) = w;
        }
}

// Shape of dq_kernel: query rows per workgroup, 32 per wave.  Eight waves
// at d = 128 (one workgroup per CU at two waves per SIMD) copy each K / V
// tile into LDS once per 256 rows instead of once per 128.
template <int D>
struct DqShape {
    static constexpr int WAVES = D == 128 ? 8 : 4;
    static constexpr int NT = 64 * WAVES;
    static constexpr int ROWS = 32 * WAVES;
    static constexpr int PER_CU = D == 128 ? 1 : 3;    // resident workgroups per CU
};

// O32: D = rowsum(dO * O) from an fp32 O (p.o32) instead of the 16-bit one
template <class T, int D, bool CAUSAL, bool O32 = false>
__global__ void __launch_bounds__(DqShape<D>::NT)
__attribute__((amdgpu_waves_per_eu(D == 128 ? 2 : 3, D == 128 ? 2 : 3))) dq_kernel(BwdParams p) {
    using G = Geo<D>;
    constexpr int ROWS = DqShape<D>::ROWS, NT = DqShape<D>::NT;
    // K and V tiles, double-buffered
    __shared__ __attribute__((aligned(16))) uint8_t ks[2][G::TILE * G::PITCH];
    __shared__ __attribute__((aligned(16))) uint8_t vs[2][G::TILE * G::PITCH];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 31, lh = lane >> 5;
    const int N = p.N;
    int hh, qb;
    if (CAUSAL) {
        causal_order(blockIdx.x, p.heads, p.nblk, p.group, hh, qb);
        qb = p.nblk - 1 - qb;                  // the last rows see the most keys
    } else {
        const int L = xcd_remap(blockIdx.x, gridDim.x);
        hh = L / p.nblk;
        qb = L - hh * p.nblk;
    }
    const int q0 = qb * ROWS, qw = q0 + 32 * wave, q = qw + li;
    const size_t head = (size_t)hh * N * D;
    const uint32_t hb = (uint32_t)N * D * 2;
    const auto rq = make_rsrc(p.q + head, hb), rk = make_rsrc(p.k + head, hb), rv = make_rsrc(p.v + head, hb);
    const auto rdo = make_rsrc(p.dout + head, hb);
    const auto ro = O32 ? make_rsrc(p.o32 + head, 2 * hb) : make_rsrc(p.o + head, hb);

    // the wave's rows as B operands: lane (li, lh) holds row q, columns 16 s + 8 lh .. +7
    u32x4_t qreg[G::NS], dreg[G::NS];
    float dsum = 0.f;
#pragma unroll
    for (int s = 0; s < G::NS; ++s) {
        const uint32_t off = (uint32_t)((q * D + 16 * s + 8 * lh) * 2);
        qreg[s] = buf_load16(rq, off);
        dreg[s] = buf_load16(rdo, off);
        if constexpr (O32)
            dsum += dot8f<T>(dreg[s], buf_load16(ro, 2 * off), buf_load16(ro, 2 * off + 16));
        else
            dsum += dot8<T>(dreg[s], buf_load16(ro, off));
    }
    dsum = sum_halves(dsum);
    const bool qok = q < N;
    if (qok && lh == 0) p.delta[(size_t)hh * N + q] = dsum;
    const float lse2 = qok ? p.lse[(size_t)hh * N + q] * kLog2e : __builtin_inff();
    const float c = p.c;

    f32x16_t acc[G::NDB];
#pragma unroll
    for (int db = 0; db < G::NDB; ++db) acc[db] = f32x16_t{};

    const int kend = CAUSAL ? min(N, q0 + ROWS) : N;
    const int nkt = (kend + G::TILE - 1) / G::TILE;
    TileRegs<D, NT> kr, vr;
    kr.load(rk, 0, tid);
    vr.load(rv, 0, tid);
    kr.store(ks[0], tid);
    vr.store(vs[0], tid);
    __syncthreads();
    for (int kt = 0; kt < nkt; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nkt;
        if (more) {                            // next tile in flight during this one
            kr.load(rk, (kt + 1) * G::TILE, tid);
            vr.load(rv, (kt + 1) * G::TILE, tid);
        }
        const uint8_t* kc = ks[cur];
        const uint8_t* vc = vs[cur];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int k0 = kt * G::TILE + 32 * sub;
            if (k0 >= N || (CAUSAL && k0 > qw + 31)) continue;   // wave-uniform: no visible key
            // S^T and dP^T: A = K / V rows (key k0 + li), B = this wave's Q / dO rows
            f32x16_t st{}, dpt{};
#pragma unroll
            for (int s = 0; s < G::NS; ++s) {
                const int off = (32 * sub + li) * G::PITCH + (16 * s + 8 * lh) * 2;
                st = mma<T>(*(const u32x4_t*)(kc + off), qreg[s], st);
                dpt = mma<T>(*(const u32x4_t*)(vc + off), dreg[s], dpt);
            }
            float ds[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = k0 + 8 * (r / 4) + 4 * lh + (r % 4);
                const bool vis = key < N && (!CAUSAL || key <= q);
                const float pr = vis ? __builtin_amdgcn_exp2f(c * st[r] - lse2) : 0.f;
                ds[r] = pr * (dpt[r] - dsum);
            }
            u32x4_t b[2];
            pack_b<T>(ds, b);
            // dQ^T += K^T dS^T
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int db = 0; db < G::NDB; ++db)
                    acc[db] = mma<T>(tr_operand<D>(kc, 32 * sub, t, 32 * db, lane), b[t], acc[db]);
        }
        // the other buffers were last read before the previous barrier
        if (more) {
            kr.store(ks[cur ^ 1], tid);
            vr.store(vs[cur ^ 1], tid);
        }
        __syncthreads();
    }
    store_rows<T, D>(p.dq + head, q, N, acc, p.scale, lh);
}

// Shape of dkdv_kernel.  At d = 128 the accumulators of dK and dV (128
// registers) and the K operand leave no room for V in registers at two waves
// per SIMD, so eight waves (256 keys) share their V rows through LDS (68 KiB
// beside the 68 KiB of Q / dO double buffers); at d = 64 four waves keep
// both K and V in registers, and with the Q / dO tiles copied straight into
// LDS (168 VGPRs) three workgroups share a CU.
template <int D>
struct DkdvShape {
    static constexpr int WAVES = D == 128 ? 8 : 4;
    static constexpr int NT = 64 * WAVES;
    static constexpr int KEYS = 32 * WAVES;        // keys per workgroup
    static constexpr bool V_LDS = D == 128;
    static constexpr bool DIRECT = D == 64;            // Q / dO tiles copied straight into LDS
    static constexpr int PER_CU = D == 128 ? 1 : 3;    // resident workgroups per CU
};

template <class T, int D, bool CAUSAL>
__global__ void __launch_bounds__(DkdvShape<D>::NT)
__attribute__((amdgpu_waves_per_eu(D == 128 ? 2 : 3, D == 128 ? 2 : 3))) dkdv_kernel(BwdParams p) {
    using G = Geo<D>;
    using S = DkdvShape<D>;
    // Q and dO tiles with their rows' LSE (base 2) and D, double-buffered
    __shared__ __attribute__((aligned(16))) uint8_t qs[2][G::TILE * G::PITCH];
    __shared__ __attribute__((aligned(16))) uint8_t dos[2][G::TILE * G::PITCH];
    __shared__ __attribute__((aligned(16))) float lses[2][G::TILE];
    __shared__ __attribute__((aligned(16))) float dls[2][G::TILE];
    // the workgroup's V rows (d = 128)
    __shared__ __attribute__((aligned(16))) uint8_t vrows[S::V_LDS ? S::KEYS * G::PITCH : 16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 31, lh = lane >> 5;
    const int N = p.N;
    int hh, kb;                                // causal: block 0 sees the most queries
    if (CAUSAL) {
        causal_order(blockIdx.x, p.heads, p.nblk_k, p.group_k, hh, kb);
    } else {
        const int L = xcd_remap(blockIdx.x, gridDim.x);
        hh = L / p.nblk_k;
        kb = L - hh * p.nblk_k;
    }
    const int k0 = kb * S::KEYS, kw = k0 + 32 * wave, key = kw + li;
    const size_t head = (size_t)hh * N * D;
    const uint32_t hb = (uint32_t)N * D * 2;
    const auto rq = make_rsrc(p.q + head, hb), rk = make_rsrc(p.k + head, hb), rv = make_rsrc(p.v + head, hb);
    const auto rdo = make_rsrc(p.dout + head, hb);
    const float* lse = p.lse + (size_t)hh * N;
    const float* delta = p.delta + (size_t)hh * N;

    // the wave's keys as B operands: lane (li, lh) holds row `key`, columns
    // 16 s + 8 lh .. +7 (V from LDS at d = 128)
    u32x4_t kreg[G::NS], vreg[S::V_LDS ? 1 : G::NS];
#pragma unroll
    for (int s = 0; s < G::NS; ++s) {
        const uint32_t off = (uint32_t)((key * D + 16 * s + 8 * lh) * 2);
        kreg[s] = buf_load16(rk, off);
        if constexpr (!S::V_LDS) vreg[s] = buf_load16(rv, off);
    }
    if constexpr (S::V_LDS) {
        // rows k0 .. k0 + KEYS - 1; rows past N read as zeros
#pragma unroll
        for (int u = 0; u < S::KEYS * D / 8 / S::NT; ++u) {
            const int i = tid + S::NT * u, row = i / (D / 8), ch = i % (D / 8);
            *(u32x4_t*)(vrows + row * G::PITCH + ch * 16) = buf_load16(rv, (uint32_t)(((k0 + row) * D + ch * 8) * 2));
        }
    }
    auto v_operand = [&](int s) -> u32x4_t {
        if constexpr (S::V_LDS)
            return *(const u32x4_t*)(vrows + (32 * wave + li) * G::PITCH + (16 * s + 8 * lh) * 2);
        else
            return vreg[s];
    };
    const float c = p.c;

    f32x16_t acck[G::NDB], accv[G::NDB];
#pragma unroll
    for (int db = 0; db < G::NDB; ++db) {
        acck[db] = f32x16_t{};
        accv[db] = f32x16_t{};
    }

    const int nqt = (N + G::TILE - 1) / G::TILE;
    const int qt0 = CAUSAL ? k0 / G::TILE : 0;
    float lpre = 0.f, dpre = 0.f;
    bool rpre = false;
    // statistics of row r of tile qt: rows past N get LSE +inf, so P = 0
    // there.  The loaded values are first used when stored, so that the
    // loads stay in flight during the tile's products.
    auto load_stats = [&](int qt) {
        if (tid < G::TILE) {
            const int r = qt * G::TILE + tid;
            rpre = r < N;
            if (rpre) {
                lpre = lse[r];
                dpre = delta[r];
            }
        }
    };
    auto store_stats = [&](int b) {
        if (tid < G::TILE) {
            lses[b][tid] = rpre ? lpre * kLog2e : __builtin_inff();
            dls[b][tid] = rpre ? dpre : 0.f;
        }
    };
    // The next Q / dO tile goes HBM -> LDS during the current one.  At d = 64
    // (S::DIRECT) the buffer unit copies it into LDS itself, in wave-sized
    // 1 KiB pieces of the padded layout (16-byte chunk c at row c / CPR,
    // chunk c % CPR of the row; the row's last chunk is padding and takes a
    // copy of its first): that frees the 16 staging registers and lets three
    // waves run per SIMD.  At d = 128 it passes through registers (TileRegs),
    // which measured faster there.
    constexpr int CPR = G::PITCH / 16, NPIECE = CPR * G::TILE / 64;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    TileRegs<D, S::NT> qr, dr;
    auto fetch_tile = [&](uint8_t* qbuf, uint8_t* dbuf, int qt) {
        if constexpr (S::DIRECT) {
            for (int b = wv; b < NPIECE; b += S::WAVES) {
                const int c = b * 64 + lane, row = c / CPR, ch = c % CPR;
                const uint32_t off = (uint32_t)(((qt * G::TILE + row) * D + (ch < CPR - 1 ? ch : 0) * 8) * 2);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rq, (__attribute__((address_space(3))) void*)(qbuf + b * 1024), 16, off, 0, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rdo, (__attribute__((address_space(3))) void*)(dbuf + b * 1024), 16, off, 0, 0, 0);
            }
        } else {
            qr.load(rq, qt * G::TILE, tid);
            dr.load(rdo, qt * G::TILE, tid);
        }
    };
    auto land_tile = [&](uint8_t* qbuf, uint8_t* dbuf) {   // register-staged copies into LDS
        if constexpr (!S::DIRECT) {
            qr.store(qbuf, tid);
            dr.store(dbuf, tid);
        }
    };
    if (qt0 < nqt) {
        fetch_tile(qs[0], dos[0], qt0);
        load_stats(qt0);
        land_tile(qs[0], dos[0]);
        store_stats(0);
    }
    __syncthreads();
    for (int qt = qt0; qt < nqt; ++qt) {
        const int cur = (qt - qt0) & 1;
        const bool more = qt + 1 < nqt;
        if (more) {                            // next tile in flight during this one
            fetch_tile(qs[cur ^ 1], dos[cur ^ 1], qt + 1);
            load_stats(qt + 1);
        }
        const uint8_t* qc = qs[cur];
        const uint8_t* dc = dos[cur];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int qs0 = qt * G::TILE + 32 * sub;
            if (qs0 >= N || (CAUSAL && qs0 + 31 < kw)) continue;   // wave-uniform: every query before every key
            // S and dP: A = Q / dO rows (query qs0 + li), B = this wave's K / V rows
            f32x16_t st{}, dpt{};
#pragma unroll
            for (int s = 0; s < G::NS; ++s) {
                const int off = (32 * sub + li) * G::PITCH + (16 * s + 8 * lh) * 2;
                st = mma<T>(*(const u32x4_t*)(qc + off), kreg[s], st);
                dpt = mma<T>(*(const u32x4_t*)(dc + off), v_operand(s), dpt);
            }
            float pr[16], ds[16];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int rl = 32 * sub + 8 * g + 4 * lh;          // local row of registers 4g .. 4g + 3
                const f32x4_t l4 = *(const f32x4_t*)(lses[cur] + rl);
                const f32x4_t d4 = *(const f32x4_t*)(dls[cur] + rl);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * g + e, qi = qs0 + 8 * g + 4 * lh + e;
                    const bool vis = !CAUSAL || key <= qi;
                    pr[r] = vis ? __builtin_amdgcn_exp2f(c * st[r] - l4[e]) : 0.f;
                    ds[r] = pr[r] * (dpt[r] - d4[e]);
                }
            }
            u32x4_t bp[2], bd[2];
            pack_b<T>(pr, bp);
            pack_b<T>(ds, bd);
            // dV^T += dO^T P,  dK^T += Q^T dS
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int db = 0; db < G::NDB; ++db) {
                    accv[db] = mma<T>(tr_operand<D>(dc, 32 * sub, t, 32 * db, lane), bp[t], accv[db]);
                    acck[db] = mma<T>(tr_operand<D>(qc, 32 * sub, t, 32 * db, lane), bd[t], acck[db]);
                }
        }
        // the other buffers were last read before the previous barrier
        if (more) {
            land_tile(qs[cur ^ 1], dos[cur ^ 1]);
            store_stats(cur ^ 1);
        }
        __syncthreads();
    }
    store_rows<T, D>(p.dk + head, key, N, acck, p.scale, lh);
    store_rows<T, D>(p.dv + head, key, N, accv, 1.0f, lh);
}

}  // namespace bwd
}  // namespace fa
