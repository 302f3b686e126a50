// FlashAttention forward kernels for gfx950 (CDNA4, wave64, MFMA).
//
// What is computed follows "FlashAttention分块计算优化Transformer显存效率":
// §1.1 (outer loop over query tiles, inner loop over key/value tiles, the
// query tile loaded once, the output tile written once), §3.2 (running
// maximum m, running sum l, correction exp(m_old - m_new) applied to l and to
// the running output), §2.2 (key tiles entirely above the diagonal are never
// loaded; tiles crossing it are masked on chip); and "Flash Attention 原理"
// (the normalisation by the merged sum at the end, and the per-row
// statistics kept for a recomputing backward pass, stored here as one fp32
// log-sum-exp per row).
//
// MI355X mapping (16-bit inputs):
//   * One workgroup = 4 waves = one 128-row query tile of one (batch, head).
//     Each wave owns 32 query rows for the whole key loop.
//   * The scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_{bf16,f16}: a lane then holds 32 key scores of ONE
//     query, so the row maximum and row sum are in-lane reductions plus one
//     permlane32 swap between the two half-waves.  The output is also
//     accumulated transposed, O^T = V^T P^T, so the per-query rescale factor
//     is a per-lane scalar and P^T feeds the second MFMA straight from
//     registers (no LDS round trip for P).
//   * The key rows of the first MFMA's A operand are loaded in a permuted
//     order (bits 2 and 3 of the row index swapped) so that each half-wave's
//     eight consecutive accumulator registers hold eight consecutive keys:
//     the P^T operand is then a plain register slice and the V^T operand one
//     16-byte LDS read.
//   * K and V tiles (tile_k x d, 16 KiB each) are double-buffered in LDS.
//     Two waves stage K (16-byte coalesced loads, XOR-swizzled rows), two
//     waves stage V and transpose it to V^T in registers (8x8 blocks) on the
//     way into LDS.  One barrier per key tile.
//   * Loads go through buffer resources bounded at the head's extent, so the
//     ragged last tile reads zeros past row N instead of faulting; those keys
//     are masked to -inf and those query rows are not stored.
//   * exp is v_exp_f32 (2^x) with log2(e) folded into the scale.
//   * Workgroups are renumbered so that the query tiles of one head run on
//     one XCD (dispatch is round-robin over the 8 XCDs): the head's K and V
//     are then re-read from that XCD's L2.  Causal launches issue the
//     longest query tiles first.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

struct BF16 {};
struct F16 {};

constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kNumXcd = 8;

// ---------------------------------------------------------------------------
// Small device helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    // raw buffer (stride 0); reads at offsets >= bytes return zero
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// v_permlane32_swap (gfx950) exchanges the upper half-wave of its first
// operand with the lower half-wave of its second.  With both operands = x,
// every lane ends up holding {its own x, x of the lane 32 away} in the two
// results (in an order that depends on the half), so the symmetric
// combinations below are the same bits in both half-waves.
__device__ __forceinline__ float max_halves(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <class T> __device__ __forceinline__ f32x16_t mma(u32x4_t a, u32x4_t b, f32x16_t c);
template <> __device__ __forceinline__ f32x16_t mma<BF16>(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x16_t mma<F16>(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// two fp32 -> two 16-bit values packed low/high, round to nearest even
template <class T> __device__ __forceinline__ uint32_t pack2(float a, float b);
template <> __device__ __forceinline__ uint32_t pack2<BF16>(float a, float b) {
    bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}
template <> __device__ __forceinline__ uint32_t pack2<F16>(float a, float b) {
    f16x2_t v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// Workgroup index -> logical tile index such that each XCD receives a
// contiguous range of logical tiles (workgroup b runs on XCD b % 8).
__device__ __forceinline__ int xcd_remap(int bid, int total) {
    const int xcd = bid % kNumXcd, slot = bid / kNumXcd;
    const int q = total / kNumXcd, r = total % kNumXcd;
    return xcd * q + (xcd < r ? xcd : r) + slot;
}

// Tile class counts, with the precedence causal-masked > ragged > full.
template <int BQ, int BK, bool CAUSAL>
__device__ void add_tile_counts(unsigned long long* counters, int qt0, int jend, int N) {
    const int nk = (N + BK - 1) / BK;
    unsigned long long full = 0, masked = 0, ragged = 0;
    for (int j = 0; j < jend; ++j) {
        const int k0 = j * BK, k1 = min(k0 + BK, N) - 1;
        if (CAUSAL && k1 > qt0) ++masked;
        else if (k1 - k0 + 1 < BK) ++ragged;
        else ++full;
    }
    atomicAdd(counters + 0, (unsigned long long)jend);
    atomicAdd(counters + 1, full);
    atomicAdd(counters + 2, masked);
    atomicAdd(counters + 3, ragged);
    atomicAdd(counters + 4, (unsigned long long)(nk - jend));
}

struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int N;
    int tiles_q;        // ceil(N / BQ)
    int total;          // B * H * tiles_q
    float c;            // |scale| * log2(e), at least FLT_MIN
    uint32_t qsign;     // 0x80008000 to negate Q (negative scale), else 0
    unsigned long long* counters;
};

// ---------------------------------------------------------------------------
// 16-bit kernel (bf16 / fp16)
// ---------------------------------------------------------------------------

template <class T, int D, bool CAUSAL, bool OUT_F32, bool COUNT>
struct Fwd16 {
    static constexpr int BQ = 128;                 // query rows per workgroup
    static constexpr int WAVES = 4;
    static constexpr int OCC = 2;                  // waves per SIMD (<= 256 VGPRs)
    static constexpr int NT = 64 * WAVES;
    static constexpr int BK = 8192 / D;            // keys per tile: tile_k x d = 16 KiB
    static constexpr int KCH = D / 8;              // 16-byte chunks per K row
    static constexpr int VCH = BK / 8;             // 16-byte chunks per V^T row
    static constexpr int NMB = BK / 32;            // 32-key blocks per tile
    static constexpr int NS = D / 16;              // k-steps of Q K^T
    static constexpr int NDB = D / 32;             // 32-wide d blocks of O^T
    static constexpr int KBYTES = BK * D * 2;
    static constexpr int BUFBYTES = 2 * KBYTES;    // K + V^T
    static constexpr int LDS = 2 * BUFBYTES;       // double buffered
    static_assert(BK % 32 == 0 && D % 32 == 0, "tile shape");
    static_assert((BK / 8) * (D / 8) == 128, "V staging assumes 128 threads");

    // row permutation of the K operand: swap bits 2 and 3
    static __device__ __forceinline__ int perm_row(int r) {
        return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
    }
    // XOR swizzles of the 16-byte chunk index (conflict-free 16-lane reads)
    static __device__ __forceinline__ int swz_k(int r) {
        return D == 128 ? (perm_row(r) & 15) : ((r >> 1) & 7);
    }
    static __device__ __forceinline__ int swz_v(int d) {
        return D == 128 ? (((d >> 1) ^ (d >> 4)) & 7) : ((d ^ (d >> 3)) & 15);
    }

    static __device__ void run(const FwdParams& p) {
        __shared__ __attribute__((aligned(16))) uint8_t smem[LDS];
        const int tid = threadIdx.x;
        const int wave = tid >> 6, lane = tid & 63;
        const int li = lane & 31, lh = lane >> 5;
        const int N = p.N;

        const int L = xcd_remap(blockIdx.x, p.total);
        const int hh = L / p.tiles_q;
        int qi = L - hh * p.tiles_q;
        if (CAUSAL) qi = p.tiles_q - 1 - qi;
        const int qt0 = qi * BQ;
        const int q0w = qt0 + wave * 32;
        const int qrow = q0w + li;

        const size_t head_elems = (size_t)hh * N * D;
        const uint32_t head_bytes = (uint32_t)N * D * 2;
        const auto rq = make_rsrc((const uint8_t*)p.q + head_elems * 2, head_bytes);
        const auto rk = make_rsrc((const uint8_t*)p.k + head_elems * 2, head_bytes);
        const auto rv = make_rsrc((const uint8_t*)p.v + head_elems * 2, head_bytes);

        // Q^T operand: lane (li, lh) holds Q[qrow][16 s + 8 lh .. +7]
        u32x4_t qreg[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            qreg[s] = buf_load16(rq, (uint32_t)(qrow * D + 16 * s + 8 * lh) * 2);
            qreg[s] ^= p.qsign;
        }

        const int nk = (N + BK - 1) / BK;
        const int jend = CAUSAL ? (min(qt0 + BQ, N) - 1) / BK + 1 : nk;

        // staging roles: threads 0..127 stage K, 128..255 stage V
        const bool stage_k = tid < 128;
        const int st = tid & 127;
        u32x4_t stg[8];

        auto gload = [&](int j) {
            const int k0 = j * BK;
            if (stage_k) {
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int id = st + 128 * u, row = id / KCH, c = id % KCH;
                    stg[u] = buf_load16(rk, (uint32_t)((k0 + row) * D + c * 8) * 2);
                }
            } else {
                const int kg = st / (D / 8), dc = st % (D / 8);
#pragma unroll
                for (int r = 0; r < 8; ++r)
                    stg[r] = buf_load16(rv, (uint32_t)((k0 + 8 * kg + r) * D + 8 * dc) * 2);
            }
        };
        auto lstore = [&](int buf) {
            uint8_t* kb = smem + buf * BUFBYTES;
            uint8_t* vb = kb + KBYTES;
            if (stage_k) {
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int id = st + 128 * u, row = id / KCH, c = id % KCH;
                    *(u32x4_t*)(kb + row * (D * 2) + ((c ^ swz_k(row)) << 4)) = stg[u];
                }
            } else {
                // 8 keys x 8 d  ->  8 d-rows x 8 keys (V^T)
                const int kg = st / (D / 8), dc = st % (D / 8);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                    u32x4_t w;
#pragma unroll
                    for (int kp = 0; kp < 4; ++kp)
                        w[kp] = __builtin_amdgcn_perm(stg[2 * kp + 1][e >> 1], stg[2 * kp][e >> 1], sel);
                    const int d = 8 * dc + e;
                    *(u32x4_t*)(vb + d * (BK * 2) + ((kg ^ swz_v(d)) << 4)) = w;
                }
            }
        };

        f32x16_t acc[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] = f32x16_t{};
        float m = -__builtin_inff(), l = 0.f;
        const float c = p.c;

        gload(0);
        lstore(0);
        __syncthreads();

        for (int j = 0; j < jend; ++j) {
            const int buf = j & 1;
            if (j + 1 < jend) gload(j + 1);
            const uint8_t* kb = smem + buf * BUFBYTES;
            const uint8_t* vb = kb + KBYTES;
            const int k0 = j * BK;
            const bool active = (!CAUSAL || k0 <= q0w + 31) && q0w < N;
            if (active) {
                // S^T = K Q^T : block mb holds keys k0 + 32 mb + ...
                f32x16_t s[NMB];
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb) {
                    s[mb] = f32x16_t{};
                    const int row = 32 * mb + perm_row(li);
                    const uint8_t* rp = kb + row * (D * 2);
                    const int sw = swz_k(row);
#pragma unroll
                    for (int ks = 0; ks < NS; ++ks) {
                        const u32x4_t a = *(const u32x4_t*)(rp + (((2 * ks + lh) ^ sw) << 4));
                        s[mb] = mma<T>(a, qreg[ks], s[mb]);
                    }
                }
                // register r of block mb holds key k0 + 32 mb + 16 (r >> 3) + 8 lh + (r & 7)
                const bool need_mask = (CAUSAL && k0 + BK - 1 > q0w) || (k0 + BK > N);
                if (need_mask) {
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int key = k0 + 32 * mb + 16 * (r >> 3) + 8 * lh + (r & 7);
                            const bool hide = (CAUSAL && key > qrow) || key >= N;
                            if (hide) s[mb][r] = -__builtin_inff();
                        }
                }
                float mx = -__builtin_inff();
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[mb][r]);
                mx = max_halves(mx);
                const float mnew = __builtin_fmaxf(m, mx);
                const float alpha = __builtin_amdgcn_exp2f((m - mnew) * c);
                const float mc = mnew * c;
                m = mnew;
                float ls = 0.f;
                u32x4_t pk[2 * NMB];
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int w = 0; w < 4; ++w) {
                            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mb][8 * t + 2 * w], c, -mc));
                            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mb][8 * t + 2 * w + 1], c, -mc));
                            ls += p0 + p1;
                            pk[2 * mb + t][w] = pack2<T>(p0, p1);
                        }
                l = l * alpha + ls;
                if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
                    for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
                }
                // O^T += V^T P^T : k-step (mb, t) covers keys k0 + 32 mb + 16 t + 8 lh + 0..7
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const int d = 32 * db + li;
                    const uint8_t* rp = vb + d * (BK * 2);
                    const int sw = swz_v(d);
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                        for (int t = 0; t < 2; ++t) {
                            const u32x4_t a = *(const u32x4_t*)(rp + (((4 * mb + 2 * t + lh) ^ sw) << 4));
                            acc[db] = mma<T>(a, pk[2 * mb + t], acc[db]);
                        }
                }
            }
            if (j + 1 < jend) lstore(buf ^ 1);
            __syncthreads();
        }

        // epilogue: O = O_running / l, LSE = ln(sum exp(scale * S))
        const float lt = sum_halves(l);
        if (q0w < N && qrow < N) {
            const float inv = 1.0f / lt;
            const size_t orow = head_elems + (size_t)qrow * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int d0 = 32 * db + 8 * jj + 4 * lh;
                    const float o0 = acc[db][4 * jj + 0] * inv, o1 = acc[db][4 * jj + 1] * inv;
                    const float o2 = acc[db][4 * jj + 2] * inv, o3 = acc[db][4 * jj + 3] * inv;
                    if (OUT_F32) {
                        *(f32x4_t*)((float*)p.o + orow + d0) = f32x4_t{o0, o1, o2, o3};
                    } else {
                        *(u32x2_t*)((uint16_t*)p.o + orow + d0) = u32x2_t{pack2<T>(o0, o1), pack2<T>(o2, o3)};
                    }
                }
            if (lh == 0) p.lse[(size_t)hh * N + qrow] = (m * c + __log2f(lt)) * kLn2;
        }
        if (COUNT && tid == 0) add_tile_counts<BQ, BK, CAUSAL>(p.counters, qt0, jend, N);
    }
};

// ---------------------------------------------------------------------------
// fp32 kernel: fp32 MFMA (v_mfma_f32_32x32x2_f32), 64 x 64 tiles
// ---------------------------------------------------------------------------

template <int D, bool CAUSAL, bool COUNT>
struct Fwd32 {
    static constexpr int BQ = 64;                  // 2 waves x 32 query rows
    static constexpr int WAVES = 2;
    static constexpr int OCC = 1;
    static constexpr int NT = 64 * WAVES;
    static constexpr int BK = 64;
    static constexpr int NMB = BK / 32;
    static constexpr int NDB = D / 32;
    static constexpr int PITCH = D + 4;            // floats per LDS row (bank spread)
    static constexpr int LDS = 2 * BK * PITCH * 4; // K and V, single buffered
    static constexpr int CH = BK * D / 4;          // 16-byte chunks per tile

    static __device__ __forceinline__ int perm_row(int r) {
        return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
    }

    static __device__ void run(const FwdParams& p) {
        __shared__ __attribute__((aligned(16))) uint8_t smem[LDS];
        float* ks = (float*)smem;
        float* vs = ks + BK * PITCH;
        const int tid = threadIdx.x;
        const int wave = tid >> 6, lane = tid & 63;
        const int li = lane & 31, lh = lane >> 5;
        const int N = p.N;

        const int L = xcd_remap(blockIdx.x, p.total);
        const int hh = L / p.tiles_q;
        int qi = L - hh * p.tiles_q;
        if (CAUSAL) qi = p.tiles_q - 1 - qi;
        const int qt0 = qi * BQ;
        const int q0w = qt0 + wave * 32;
        const int qrow = q0w + li;

        const size_t head_elems = (size_t)hh * N * D;
        const uint32_t head_bytes = (uint32_t)N * D * 4;
        const auto rq = make_rsrc((const uint8_t*)p.q + head_elems * 4, head_bytes);
        const auto rk = make_rsrc((const uint8_t*)p.k + head_elems * 4, head_bytes);
        const auto rv = make_rsrc((const uint8_t*)p.v + head_elems * 4, head_bytes);

        // Q^T operand for k-step s: Q[qrow][2 s + lh]
        float qreg[D / 2];
#pragma unroll
        for (int s4 = 0; s4 < D / 8; ++s4) {
            // 4 consecutive k-steps need d = 8 s4 + 2 t + lh, t = 0..3
            const u32x4_t lo = buf_load16(rq, (uint32_t)(qrow * D + 8 * s4) * 4);
            const u32x4_t hi = buf_load16(rq, (uint32_t)(qrow * D + 8 * s4 + 4) * 4);
            const uint32_t sgn = p.qsign ? 0x80000000u : 0u;
            qreg[4 * s4 + 0] = __uint_as_float((lh ? lo[1] : lo[0]) ^ sgn);
            qreg[4 * s4 + 1] = __uint_as_float((lh ? lo[3] : lo[2]) ^ sgn);
            qreg[4 * s4 + 2] = __uint_as_float((lh ? hi[1] : hi[0]) ^ sgn);
            qreg[4 * s4 + 3] = __uint_as_float((lh ? hi[3] : hi[2]) ^ sgn);
        }

        const int nk = (N + BK - 1) / BK;
        const int jend = CAUSAL ? (min(qt0 + BQ, N) - 1) / BK + 1 : nk;

        f32x16_t acc[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] = f32x16_t{};
        float m = -__builtin_inff(), l = 0.f;
        const float c = p.c;

        for (int j = 0; j < jend; ++j) {
            const int k0 = j * BK;
            for (int id = tid; id < CH; id += NT) {
                const int row = id / (D / 4), c4 = id % (D / 4);
                const uint32_t off = (uint32_t)((k0 + row) * D + 4 * c4) * 4;
                *(u32x4_t*)(ks + row * PITCH + 4 * c4) = buf_load16(rk, off);
                *(u32x4_t*)(vs + row * PITCH + 4 * c4) = buf_load16(rv, off);
            }
            __syncthreads();
            const bool active = (!CAUSAL || k0 <= q0w + 31) && q0w < N;
            if (active) {
                f32x16_t s[NMB];
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb) {
                    s[mb] = f32x16_t{};
                    const float* rp = ks + (32 * mb + perm_row(li)) * PITCH + lh;
#pragma unroll
                    for (int st = 0; st < D / 2; ++st)
                        s[mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(rp[2 * st], qreg[st], s[mb], 0, 0, 0);
                }
                const bool need_mask = (CAUSAL && k0 + BK - 1 > q0w) || (k0 + BK > N);
                if (need_mask) {
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int key = k0 + 32 * mb + 16 * (r >> 3) + 8 * lh + (r & 7);
                            if ((CAUSAL && key > qrow) || key >= N) s[mb][r] = -__builtin_inff();
                        }
                }
                float mx = -__builtin_inff();
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[mb][r]);
                mx = max_halves(mx);
                const float mnew = __builtin_fmaxf(m, mx);
                const float alpha = __builtin_amdgcn_exp2f((m - mnew) * c);
                const float mc = mnew * c;
                m = mnew;
                float ls = 0.f;
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        s[mb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mb][r], c, -mc));
                        ls += s[mb][r];
                    }
                l = l * alpha + ls;
#pragma unroll
                for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
                // O^T += V^T P^T, one key per half-wave per k-step
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = 32 * mb + 16 * (r >> 3) + 8 * lh + (r & 7);
#pragma unroll
                        for (int db = 0; db < NDB; ++db)
                            acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[key * PITCH + 32 * db + li],
                                                                           s[mb][r], acc[db], 0, 0, 0);
                    }
            }
            __syncthreads();
        }

        const float lt = sum_halves(l);
        if (q0w < N && qrow < N) {
            const float inv = 1.0f / lt;
            const size_t orow = head_elems + (size_t)qrow * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int d0 = 32 * db + 8 * jj + 4 * lh;
                    *(f32x4_t*)((float*)p.o + orow + d0) =
                        f32x4_t{acc[db][4 * jj] * inv, acc[db][4 * jj + 1] * inv,
                                acc[db][4 * jj + 2] * inv, acc[db][4 * jj + 3] * inv};
                }
            if (lh == 0) p.lse[(size_t)hh * N + qrow] = (m * c + __log2f(lt)) * kLn2;
        }
        if (COUNT && tid == 0) add_tile_counts<BQ, BK, CAUSAL>(p.counters, qt0, jend, N);
    }
};

template <class K>
__global__ void __launch_bounds__(K::NT) __attribute__((amdgpu_waves_per_eu(K::OCC, K::OCC))) fwd_kernel(FwdParams p) {
    K::run(p);
}

}  // namespace fa
