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
//   * One workgroup = one query tile of one (batch, head): 8 waves / 256 rows
//     without a mask at d = 128, 4 waves / 128 rows causal (two workgroups
//     per CU) and at d = 64 (three per CU).  Each wave owns 32 query rows
//     for the whole key loop.
//   * The scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_{bf16,f16}: a lane then holds 32 key scores of ONE
//     query, so the row sums are in-lane reductions plus one permlane32
//     swap between the two half-waves.  The output is also accumulated
//     transposed, O^T = V^T P^T, so the per-query rescale factor is a
//     per-lane scalar and P^T feeds the second MFMA straight from registers
//     (no LDS round trip for P).
//   * The key rows of the first MFMA's A operand are loaded in a permuted
//     order (bits 2 and 3 of the row index swapped) so that each half-wave's
//     eight consecutive accumulator registers hold eight consecutive keys:
//     the P^T operand is then a plain register slice.
//   * K and V tiles (tile_k x d, 16 KiB each at d = 128) are double-buffered
//     in LDS and filled by the buffer unit's direct-to-LDS loads, spread over
//     the MFMA schedule; V^T operands come from row-major V through the
//     transposing LDS read.  One barrier per key tile.
//   * Loads go through buffer resources bounded at the head's extent, so the
//     ragged last tile reads zeros past row N instead of faulting; those keys
//     are masked to -inf and those query rows are not stored.
//   * exp is v_exp_f32 (2^x) with log2(e) folded into the scale.
//   * Workgroups are renumbered so that the query tiles of one head run on
//     one XCD (dispatch is round-robin over the 8 XCDs): the head's K and V
//     are then re-read from that XCD's L2.  Causal launches issue query
//     tiles longest first across all heads, which balances the CUs' loads.
//   * At d = 128, launches with more query tiles than workgroup slots run a
//     persistent variant (Fwd16P): one workgroup per CU runs the key loops
//     of its query tiles back to back as one software pipeline, so the
//     pipeline does not drain and refill between query tiles.  Under the
//     mask the persistent variant takes pairs of 256-row query tiles
//     (i, T - 1 - i) of equal total cost.
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
    float m;
    asm volatile("v_max_f32 %0, %1, %2" : "=v"(m) : "v"(__uint_as_float(r[0])), "v"(__uint_as_float(r[1])));
    return m;
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
    int heads;          // B * H
    int tiles_q;        // ceil(N / BQ)
    int total;          // heads * tiles_q
    int group;          // heads per group of the causal tile order
    float c;            // |scale| * log2(e), at least FLT_MIN
    uint32_t qsign;     // 0x80008000 to negate Q (negative scale), else 0
    unsigned long long* counters;
    int splits;         // split-KV launches: key ranges per query tile
    int split_len;      // keys per range (a multiple of the key tile)
};

// Workgroup index -> (head, query tile).
//
// Without a mask every query tile costs the same; each XCD receives a
// contiguous range of logical tiles (head-major), so that a head's K and V
// are re-read from one L2.
//
// Under the causal mask query tile i costs i + 1 key-tile steps.  The
// dispatcher starts workgroups in index order as slots free up, so tiles are
// issued longest first (by rank = tiles_q - 1 - i), which ends the launch
// with the short ones.  With a head count divisible by 8, XCD x (which runs
// workgroups b = x mod 8) owns heads x, x + 8, ... and takes them in groups
// of `group` heads, rank-major inside a group: a group's tiles fill the
// XCD's workgroup slots, and only its few heads' K and V are live in the L2
// at a time.  Otherwise tiles go rank-major across all heads.
struct TileId {
    int hh, qi;
};
template <bool CAUSAL>
__device__ __forceinline__ TileId tile_of(int bid, const FwdParams& p) {
    if (!CAUSAL) {
        const int L = xcd_remap(bid, p.total);
        const int hh = L / p.tiles_q;
        return {hh, L - hh * p.tiles_q};
    }
    if (p.heads % kNumXcd == 0) {
        const int x = bid % kNumXcd, s = bid / kNumXcd;   // s < heads / 8 * tiles_q
        const int hpx = p.heads / kNumXcd;
        const int gsz = p.group * p.tiles_q;
        const int g = s / gsz, w = s - g * gsz;
        const int gg = min(p.group, hpx - g * p.group);   // heads in this group
        const int rank = w / gg;
        return {(g * p.group + w - rank * gg) * kNumXcd + x, p.tiles_q - 1 - rank};
    }
    const int rank = bid / p.heads;
    return {bid - rank * p.heads, p.tiles_q - 1 - rank};
}

// Heads per group of a causal order like the one above: enough for the
// group's blocks to fill the workgroup slots of one XCD twice, at most the
// XCD's heads (the backward's block orders; measured there against groups of
// 1, 2 and all of an XCD's heads).
inline int causal_group(int heads, int tiles_q, int slots_per_xcd) {
    if (heads % kNumXcd != 0) return 1;
    const int g = (2 * slots_per_xcd + tiles_q - 1) / tiles_q;
    const int hpx = heads / kNumXcd;
    return g < 1 ? 1 : (g > hpx ? hpx : g);
}

// Heads per group of the 16-bit per-tile forward's causal order: 16, or all
// of an XCD's heads when it has fewer.  Smaller groups leave the last
// group's long tiles running alone at the end (4096 rows, 64 heads: groups of
// 2 heads); larger ones spread each head's K and V reuse out of the L2.  In
// interleaved A/B runs 16 was the best or within noise of it at every shape
// measured (d = 64: 1000 rows x 512 heads, 2048 x 512, 4096 x 64,
// 512 x 1024, 2000 x 128; d = 128: 3800 x 64, 1000 x 256), 0-6% ahead of
// groups sized to fill the slots twice.
inline int fwd_causal_group(int heads) {
    if (heads % kNumXcd != 0) return 1;
    return min(16, heads / kNumXcd);
}

// ---------------------------------------------------------------------------
// 16-bit kernel (bf16 / fp16)
//
// One workgroup = a query tile of one (batch, head), 32 query rows per wave
// for the whole key loop (8 waves without a mask, 4 causal: two waves per
// SIMD either way).
// Key tiles are 64 rows.
//
// Per key tile t a wave does three things: the scores S_t = K_t Q^T (16 MFMA
// at d = 128), the softmax of S_t (VALU), and O += V_t^T P_t^T (16 MFMA).
// They are software-pipelined one tile apart, so that iteration j issues the
// score MFMAs of tile j+1 and the output MFMAs of tile j-1 while the VALU
// works on the softmax of tile j: the three streams are independent within an
// iteration, and the MFMAs are interleaved one by one with the softmax
// instructions (a wave issues its own VALU work under a running MFMA).
//
// K and V tiles are copied HBM -> LDS by the buffer unit directly (no VGPR
// staging), double-buffered: iteration j reads K_{j+1} and V_{j-1} and fills
// the other halves with K_{j+2} and V_j, one 16-byte copy per thread every
// few MFMA slots; one barrier per iteration.  K rows are stored with their
// 16-byte chunks XOR-swizzled by row so that the 16-byte operand reads of 16
// lanes hit distinct banks; V is stored row-major (swizzled for its own
// access pattern) and read transposed with ds_read_b64_tr_b16, which hands
// every lane four consecutive keys of one head-dimension column -- the V^T
// operand of the second product.
//
// Softmax against a reference.  The running maximum of the online softmax
// only serves to keep the exponentials in range: any per-row reference r
// gives the same O and log-sum-exp, as long as numerator and denominator
// share it and no term overflows.  So a row keeps its reference, and its
// running output unscaled, through every tile whose terms exp2(c s - r) sum
// to at most 2^15 (which bounds every term and keeps fp16 terms finite) and
// to at most the row's running sum.  Any other tile -- always the first,
// whose reference starts at -FLT_MAX -- takes the slow path: the reference
// is raised to the row's maximum so far, the running output and sum are
// rescaled by exp2(r_old - r_new), and the tile's terms are recomputed.  The
// tile maximum is never computed on the fast path.
//
// The second condition is for accuracy, not range: the terms are rounded to
// 16 bits for the output MFMA (relative error up to 2^-8 in bf16) while the
// sum takes them in fp32.  A term that ends up dominating its row therefore
// always passes through the slow path, where it becomes exactly 1 (or a
// power of two after later rescales) and is rounded without error; a term
// that never triggers the slow path is at most the running sum before it,
// hence at most half of the row's final sum.
// ---------------------------------------------------------------------------

typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2_t lds_read_tr(const uint8_t* p) {
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t*)(__attribute__((address_space(3))) uint8_t*)p);
    return __builtin_bit_cast(u32x2_t, v);
}

// keeps a value's computation at this point of the instruction stream: the
// compiler may not sink it past here (the MFMA interleave depends on it)
template <class X> __device__ __forceinline__ void pin(X& x) { asm volatile("" : "+v"(x)); }
// the value of a wave-uniform x, held in SGPRs from this point on
template <class X> __device__ __forceinline__ X pin_s(X x) {
    asm volatile("" : "+s"(x));
    return x;
}
// A store to global memory.  Pointers that went through pin_s have lost
// their address space; a generic (flat) store counts on the LDS counter as
// well, and inside the key loop it would make every LDS operand wait a full
// drain of that counter.
template <class X> __device__ __forceinline__ void gstore(void* p, const X& v) {
    *(__attribute__((address_space(1))) X*)p = v;
}

template <bool B> struct BoolTag { static constexpr bool value = B; };
template <int I> struct IntTag { static constexpr int value = I; };

// f(IntTag<I>{}) for I = B .. E-1, unrolled by construction (the loop bodies
// here are too large for the optimiser's unroll limits)
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(IntTag<B>{});
        static_for<B + 1, E>(f);
    }
}

// WQ (waves per workgroup, 0 = the default below) and BKT (keys per tile)
// select other tile shapes; the library builds the defaults for every type
// and a tile-size sweep (bf16, d = 128, no mask) besides.
// SPLIT: a split-KV launch (fp32 output): workgroup b takes one query tile
// over one range of p.split_len keys and writes that range's partial output
// and log-sum-exp, which a second kernel merges.  Under the causal mask a
// range may hold no key visible to a row (or to the whole tile): that row's
// partial is O = 0 with LSE = -inf, which the merge weights by exp(-inf) = 0.
template <class T, int D, bool CAUSAL, bool OUT_F32, bool COUNT, int WQ = 0, int BKT = 64, bool SPLIT = false>
struct Fwd16 {
    // Eight waves (256 query rows, one workgroup per CU) share each K / V
    // tile copy without a mask at d = 128: half the L2 -> LDS traffic of
    // four.  Causal launches keep four waves (128 rows, two workgroups per
    // CU): their waves' work differs along the diagonal, and a smaller
    // workgroup waits less at its barriers for the wave with the most keys
    // (under the longest-first tile order eight waves measure the same).  At
    // d = 64 a wave needs about 165 registers, so three waves fit on a SIMD:
    // four-wave workgroups, three per CU, under either mask -- a score costs
    // half the matrix work of d = 128 but the same softmax work, and the third
    // wave keeps more VALU work in flight beside the matrix cores.
    static constexpr int WAVES = WQ ? WQ : (D == 64 || CAUSAL ? 4 : 8);
    static constexpr int BQ = 32 * WAVES;          // query rows per workgroup
    static constexpr int OCC = D == 64 && WAVES == 4 ? 3 : 2;   // waves per SIMD
    static constexpr int RESIDENT = 4 * OCC / WAVES;   // workgroups per CU
    static constexpr int NT = 64 * WAVES;
    static constexpr int BK = BKT;                 // keys per tile
    static constexpr int ROWB = 2 * D;             // bytes per K / V row
    static constexpr int TILEB = BK * ROWB;        // bytes per K or V tile
    static constexpr int NS = D / 16;              // k-steps of K Q^T per 32-key block
    static constexpr int NDB = D / 32;             // 32-row d blocks of O^T
    static constexpr int NMB = BK / 32;            // 32-key blocks per tile
    static constexpr int NKS = BK / 16;            // k-steps of V^T P^T per tile
    static constexpr int NPV = NDB * NKS;          // output MFMAs per tile
    static constexpr int NQK = NMB * NS;           // score MFMAs per tile
    static constexpr int NSLOT = NPV + NQK;        // one MFMA per slot
    static constexpr int NV = BK / 2;              // scores per lane per tile
    static constexpr int LOADS = TILEB / (NT * 16);// 16-byte copies per thread per tile
    static constexpr int PD = 3;                   // operand prefetch distance (slots)
    // issue a slot's LDS operand read before its softmax stages (measured
    // ~1% faster with four waves, ~1% slower with eight)
    static constexpr bool READ_FIRST = WAVES == 4;
    static constexpr int LDS = 4 * TILEB;
    static_assert(D == 64 || D == 128, "head dimension");
    static_assert(LOADS >= 1 && TILEB % (NT * 16) == 0, "tile copy");
    static_assert(!SPLIT || (OUT_F32 && !COUNT), "split-KV partials: fp32 output, no counters");

    // K row permutation: swap bits 2 and 3, so that each half-wave's eight
    // consecutive score registers hold eight consecutive keys
    static __device__ __forceinline__ int perm_row(int r) {
        return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
    }
    // chunk swizzles (16-byte chunk index XOR f(row))
    static __device__ __forceinline__ int fk(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
    static __device__ __forceinline__ int fv(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

    struct Lane {
        int koff[NS];       // K operand byte offsets within a tile, per k-step
        int voff[NDB];      // V^T operand byte offsets within a tile, per d block
    };

    // Per-lane source offset (within a tile) of this lane's u-th 16-byte
    // copy.  A thread's copies are WAVES KiB apart in LDS; when that is a
    // multiple of 16 rows (every default shape) the swizzle of the row is the
    // same for all of them and one offset serves all.
    static constexpr bool SAME_SWIZZLE = (WAVES * 1024 / ROWB) % 16 == 0;
    template <bool ISK>
    static __device__ __forceinline__ uint32_t copy_offset(int wave, int lane, int u = 0) {
        const int off = (u * WAVES + wave) * 1024 + lane * 16;
        const int row = off / ROWB, pos = (off % ROWB) >> 4;
        const int chunk = pos ^ (ISK ? fk(row) : fv(row));
        return (uint32_t)(row * ROWB + chunk * 16);
    }
    // The u-th of a thread's LOADS 16-byte copies of one tile HBM -> LDS.
    // r is a buffer resource based at the tile's first row whose extent is
    // what is left of the head from there (zero for a tile past the end);
    // off is the thread's byte offset inside the tile.  The buffer unit
    // range-checks the VGPR offset against that extent, so rows past N read
    // as zeros.
    static __device__ __forceinline__ void copy_part(__amdgpu_buffer_rsrc_t r, uint8_t* lbuf, int wave,
                                                     uint32_t off, int u) {
        const int blk = u * WAVES + wave;              // 1 KiB block of the tile
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void*)(lbuf + blk * 1024), 16, off, 0, 0, 0);
    }

    static __device__ __forceinline__ u32x4_t k_operand(const uint8_t* kb, const Lane& ln, int mb, int ks) {
        return *(const u32x4_t*)(kb + ln.koff[ks] + 32 * mb * ROWB);
    }
    static __device__ __forceinline__ u32x4_t v_operand(const uint8_t* vb, const Lane& ln, int db, int kt) {
        const uint8_t* p = vb + ln.voff[db] + 16 * kt * ROWB;
        const u32x2_t a = lds_read_tr(p), b = lds_read_tr(p + 4 * ROWB);
        return u32x4_t{a[0], a[1], b[0], b[1]};
    }

    // The MFMA of slot i: slots [0, NPV) are O^T += V^T P^T (k-step major, so
    // consecutive slots go to different accumulators), the rest S^T = K Q^T.
    static __device__ __forceinline__ void slot_mfma(int i, u32x4_t a, f32x16_t* acc, f32x16_t* snext,
                                                     const u32x4_t* pprev, const u32x4_t* qreg) {
        if (i < NPV) {
            const int kt = i / NDB, db = i % NDB;
            acc[db] = mma<T>(a, pprev[kt], acc[db]);
        } else {
            const int q = i - NPV, ks = q / NMB, mb = q % NMB;
            snext[mb] = mma<T>(a, qreg[ks], ks == 0 ? f32x16_t{} : snext[mb]);
        }
    }
    static __device__ __forceinline__ u32x4_t slot_operand(int i, const uint8_t* kb, const uint8_t* vb,
                                                           const Lane& ln) {
        if (i < NPV) return v_operand(vb, ln, i % NDB, i / NDB);
        const int q = i - NPV;
        return k_operand(kb, ln, q % NMB, q / NMB);
    }

    // softmax state of one lane (one query row; both half-waves hold it)
    struct Soft {
        float mc;      // reference maximum times c (base-2 exponent units)
        float l;       // running sum of the row's terms (previous tiles, both halves)
        float lt;      // this tile's sum of this half-wave's terms
        float meff;    // mc, or +inf when this iteration has no tile (terms are 0)
    };

    // The softmax of a tile turns each score s into the term
    // exp2(c s - mc) against the row's reference mc, in three stages one or
    // two MFMA slots apart (so no instruction waits on the one before it):
    //   A  x = c s - mc for two scores                      (2 fma)
    //   B  p = 2^x                                          (2 exp)
    //   C  pack the two terms to 16 bits, add them to the tile sum
    //                                                       (cvt, 2 add)
    // Pair k (scores 2k, 2k+1) starts at slot pair_slot(k).  Its stage C
    // rewrites the term registers of k-step k/4, which the output MFMAs of
    // slots [NDB (k/4), NDB (k/4 + 1)) read first.
    static constexpr int NPAIR = NV / 2;
    static constexpr int DB_ = D == 128 ? 1 : 0;     // stage B delay (slots)
    static constexpr int DC_ = D == 128 ? 2 : 1;     // stage C delay (slots)
    static constexpr int P_FIRST = D == 128 ? 2 : 1;
    static constexpr int P_LAST = NSLOT - 1 - DC_;
    static constexpr int pair_slot(int k) { return P_FIRST + ((P_LAST - P_FIRST) * k) / (NPAIR - 1); }
    static constexpr bool terms_after_reads() {
        for (int k = 0; k < NPAIR; ++k)
            if (pair_slot(k) + DC_ < (k / 4) * NDB + NDB) return false;
        return true;
    }
    static_assert(terms_after_reads(), "softmax would overwrite terms before the output MFMA reads them");
    // copies of the next tiles: one 16-byte copy every COPY_EVERY slots
    static constexpr int NCOPY = 2 * LOADS;
    static constexpr int COPY_EVERY = NSLOT / NCOPY;
    static_assert(COPY_EVERY >= 1 && NCOPY * COPY_EVERY <= NSLOT, "copy spread");

    // a tile whose terms sum to more than this (the sum bounds every term)
    // takes the slow path; fp16 holds terms up to 65504
    static constexpr float kTileSumLimit = 32768.0f;

    static __device__ __forceinline__ void stage_a(const f32x16_t* scur, int k, const Soft& st, float c,
                                                   float& x0, float& x1) {
        x0 = __builtin_fmaf(scur[(2 * k) / 16][(2 * k) % 16], c, -st.meff);
        x1 = __builtin_fmaf(scur[(2 * k + 1) / 16][(2 * k + 1) % 16], c, -st.meff);
        pin(x0);
        pin(x1);
    }
    static __device__ __forceinline__ void stage_b(float& x0, float& x1) {
        x0 = __builtin_amdgcn_exp2f(x0);
        x1 = __builtin_amdgcn_exp2f(x1);
        pin(x0);
        pin(x1);
    }
    static __device__ __forceinline__ void stage_c(u32x4_t* pcur, int k, Soft& st, float x0, float x1) {
        uint32_t w = pack2<T>(x0, x1);
        st.lt += x0;
        st.lt += x1;
        pin(w);
        pin(st.lt);
        pcur[k / 4][k % 4] = w;
    }

    // Slow path of a tile: lanes that need it raise their reference to the
    // larger of it and the tile's maximum; the running output and sum are
    // rescaled by the correction exp2(old - new) and the tile's terms and sum
    // are recomputed.  Other lanes keep their reference and terms (their
    // correction is 1).  keep_acc leaves the accumulators alone (they hold
    // another query tile's output when the persistent kernel starts a tile).
    static __device__ void raise_reference(const f32x16_t* scur, u32x4_t* pcur, Soft& st, float c,
                                           f32x16_t* acc, bool need, bool keep_acc = false) {
        float mx = -__builtin_inff();
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, scur[mb][r]);
        mx = max_halves(mx);
        const float nmc = need ? __builtin_fmaxf(st.mc, mx * c) : st.mc;
        const float alpha = __builtin_amdgcn_exp2f(st.mc - nmc);
        st.mc = nmc;
        st.meff = nmc;
        st.l *= alpha;
        const float aacc = keep_acc ? 1.0f : alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] *= aacc;
        float lt = 0.f;
#pragma unroll
        for (int k = 0; k < NPAIR; ++k) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(scur[(2 * k) / 16][(2 * k) % 16], c, -nmc));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(scur[(2 * k + 1) / 16][(2 * k + 1) % 16], c, -nmc));
            const uint32_t w = pack2<T>(p0, p1);
            if (need) pcur[k / 4][k % 4] = w;
            lt += p0 + p1;
        }
        if (need) st.lt = lt;
    }

    static __device__ void run(const FwdParams& p) {
        // K and V double buffers (separate arrays: the compiler then knows
        // that the buffers being read never alias the ones being filled)
        __shared__ __attribute__((aligned(1024))) uint8_t kbuf0[TILEB];
        __shared__ __attribute__((aligned(1024))) uint8_t kbuf1[TILEB];
        __shared__ __attribute__((aligned(1024))) uint8_t vbuf0[TILEB];
        __shared__ __attribute__((aligned(1024))) uint8_t vbuf1[TILEB];
        const int tid = threadIdx.x;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int lane = tid & 63;
        const int li = lane & 31, lh = lane >> 5;
        const int N = p.N;
        // Every kernel argument is read into SGPRs here, before the first
        // direct-to-LDS copy: a scalar load issued while a copy is in flight
        // could target SGPRs that the copy still reads (its buffer resource
        // or M0 source).
        void* const out = pin_s(p.o);
        float* const lse = pin_s(p.lse);
        unsigned long long* const counters = pin_s(p.counters);
        const float c = pin_s(p.c);

        TileId t;
        int split = 0;                              // key range of a split-KV launch
        if constexpr (SPLIT && CAUSAL) {
            // (query tile, head, range), longest tiles first: consecutive
            // workgroups go to different XCDs, so every XCD gets its share
            // of the long tiles (a head-major order would hand one XCD all
            // of a head's last, longest tiles)
            const int per_rank = p.heads * p.splits;
            const int rank = blockIdx.x / per_rank, rem = blockIdx.x - rank * per_rank;
            t.qi = p.tiles_q - 1 - rank;
            t.hh = rem / p.splits;
            split = rem - t.hh * p.splits;
        } else if constexpr (SPLIT) {
            // (head, query tile, range), head-major so that a head's K and V
            // are re-read from one XCD's L2
            const int L = xcd_remap(blockIdx.x, p.total * p.splits);
            const int per_head = p.tiles_q * p.splits;
            t.hh = L / per_head;
            const int rem = L - t.hh * per_head;
            t.qi = rem / p.splits;
            split = rem - t.qi * p.splits;
        } else {
            t = tile_of<CAUSAL>(blockIdx.x, p);
        }
        const int hh = t.hh;
        const int qt0 = t.qi * BQ;
        const int q0w = qt0 + wave * 32;            // first row of this wave; lane li holds row q0w + li
        const int qrow = q0w + li;

        const size_t head_elems = (size_t)hh * N * D;
        const uint32_t head_bytes = (uint32_t)N * ROWB;
        // the keys this workgroup visits: the head's, or one range of them
        const int kfirst = SPLIT ? split * p.split_len : 0;
        const int NK = SPLIT ? min(p.split_len, N - kfirst) : N;
        const uint32_t kv_bytes = (uint32_t)NK * ROWB;
        const auto rq = make_rsrc((const uint8_t*)p.q + head_elems * 2, head_bytes);
        const uint8_t* kbase = (const uint8_t*)p.k + head_elems * 2 + (size_t)kfirst * ROWB;
        const uint8_t* vbase = (const uint8_t*)p.v + head_elems * 2 + (size_t)kfirst * ROWB;

        const int nk = (NK + BK - 1) / BK;
        int jend;
        if constexpr (SPLIT && CAUSAL) {
            // the last key of the tile's last row, relative to the range
            const int kmax = min(qt0 + BQ, N) - 1 - kfirst;
            jend = kmax < 0 ? 0 : min(nk, kmax / BK + 1);
        } else {
            jend = CAUSAL ? (min(qt0 + BQ, N) - 1) / BK + 1 : nk;
        }
        // opaque to the optimiser: reasoning about the causal bound makes it
        // allocate the loop body with more registers than the CU holds
        asm volatile("" : "+s"(jend));
        // key tiles this wave computes (all of them, up to its diagonal when causal)
        int wend;
        if constexpr (SPLIT && CAUSAL) {
            const int wmax = q0w + 31 - kfirst;     // this wave's last visible key, relative
            wend = q0w < N ? (wmax < 0 ? 0 : min(jend, wmax / BK + 1)) : 0;
        } else {
            wend = q0w < N ? (CAUSAL ? min(jend, (q0w + 31) / BK + 1) : jend) : 0;
        }
        wend = __builtin_amdgcn_readfirstlane(wend);

        // (All of a wave's own LDS writes -- this zero fill, the output
        // staging -- happen while none of its direct-to-LDS copies is in
        // flight: the fill comes before the first copy, the staging after a
        // barrier that waits for every copy.  A fill issued behind the first
        // copy gave nondeterministic results.)
        // Both V buffers start as zeros: the first two iterations multiply
        // them with zero terms, and rows past N of a ragged last tile stay
        // zero whether or not the copy unit writes out-of-range rows.  The K
        // buffer that may be read before it is first filled starts as zeros
        // too, so that every score is finite.
#pragma unroll
        for (int i = tid; i < TILEB / 16; i += NT) {
            ((u32x4_t*)vbuf0)[i] = u32x4_t{0, 0, 0, 0};
            ((u32x4_t*)vbuf1)[i] = u32x4_t{0, 0, 0, 0};
            ((u32x4_t*)kbuf1)[i] = u32x4_t{0, 0, 0, 0};
        }

        // Q^T operand: lane (li, lh) holds Q[row][16 s + 8 lh .. +7]
        u32x4_t qreg[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            qreg[s] = buf_load16(rq, (uint32_t)(qrow * D + 16 * s + 8 * lh) * 2);
            qreg[s] ^= p.qsign;
        }

        Lane ln;
        {
            const int prow = perm_row(li);
            const int ks_sw = fk(prow);
#pragma unroll
            for (int ks = 0; ks < NS; ++ks) ln.koff[ks] = prow * ROWB + (((2 * ks + lh) ^ ks_sw) << 4);
            const int G = lane >> 4, s = lane & 15;
            const int fvq = D == 128 ? ((s >> 2) & 3) : ((s >> 3) & 1);
            const int y = 2 * (G & 1) + ((s & 3) >> 1);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                ln.voff[db] = (8 * lh + (s >> 2)) * ROWB + ((4 * (db ^ fvq) + y) << 4) + 8 * (s & 1);
        }

        f32x16_t acc[NDB];
        f32x16_t s0[NMB], s1[NMB];     // scores of even / odd tiles
        // packed terms: the output MFMAs of an iteration read the previous
        // tile's terms from the same registers the softmax then overwrites
        // with this tile's (each k-step's registers only after their last read)
        u32x4_t pk[NKS];
        Soft st;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] = f32x16_t{};
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) s0[mb] = s1[mb] = f32x16_t{};
#pragma unroll
        for (int kt = 0; kt < NKS; ++kt) pk[kt] = u32x4_t{0, 0, 0, 0};
        // the first tile's terms overflow against this reference, which sends
        // it through the slow path that sets the real one
        st.mc = -__FLT_MAX__;
        st.l = st.lt = 0.f;

        // this thread's byte offsets inside a K / V tile, one per copy
        const uint32_t ksrc = copy_offset<true>(wave, lane);
        const uint32_t vsrc = copy_offset<false>(wave, lane);
        uint32_t koff_c[LOADS], voff_c[LOADS];
#pragma unroll
        for (int u = 0; u < LOADS; ++u) {
            if constexpr (SAME_SWIZZLE) {
                koff_c[u] = ksrc + (uint32_t)(u * WAVES * 1024);
                voff_c[u] = vsrc + (uint32_t)(u * WAVES * 1024);
            } else {
                koff_c[u] = copy_offset<true>(wave, lane, u);
                voff_c[u] = copy_offset<false>(wave, lane, u);
            }
        }

        // prologue: K_0 into kbuf0
        {
            const auto rk0 = make_rsrc(kbase, kv_bytes);
#pragma unroll
            for (int u = 0; u < LOADS; ++u) copy_part(rk0, kbuf0, wave, koff_c[u], u);
        }

        // iteration j (see the section comment); ODD selects the buffers / arrays
        auto iteration = [&](const int j, auto odd_tag) {
            constexpr bool ODD = decltype(odd_tag)::value;
            uint8_t* kread = ODD ? kbuf0 : kbuf1;      // K_{j+1}
            uint8_t* kfill = ODD ? kbuf1 : kbuf0;      // K_{j+2}
            uint8_t* vread = ODD ? vbuf0 : vbuf1;      // V_{j-1}
            uint8_t* vfill = ODD ? vbuf1 : vbuf0;      // V_j
            f32x16_t* scur = ODD ? s1 : s0;
            f32x16_t* snext = ODD ? s0 : s1;

            __syncthreads();   // this wave's copies done (vmcnt 0), and everyone's

            // Every iteration runs the same straight-line schedule (one
            // register allocation, no divergent code paths).  Where a stream
            // has nothing to do its work is made harmless instead of skipped:
            // the softmax of an iteration without a tile of this wave uses a
            // reference of +inf, so its terms and sums are exactly 0; the
            // output MFMAs then add 0 * V (the V buffers start zeroed, every V
            // row stored later is finite data), and the score MFMAs of the
            // last iterations produce scores nobody reads.
            const bool has_sm = j >= 0 && j < wend;
            const int k0 = j * BK;
            if (has_sm) {
                const bool need_mask = (CAUSAL && kfirst + k0 + BK - 1 > q0w) || (k0 + BK > NK);
                if (need_mask) {
                    // register r of block mb holds key k0 + 8 lh + kk with the
                    // constant kk below; it is visible iff kk <= lim
                    int lim = NK - 1 - k0 - 8 * lh;
                    if (CAUSAL) lim = min(lim, qrow - kfirst - k0 - 8 * lh);
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int kk = 32 * mb + 16 * (r >> 3) + (r & 7);
                            scur[mb][r] = kk > lim ? -__builtin_inff() : scur[mb][r];
                        }
                }
            }
            st.meff = has_sm ? st.mc : __builtin_inff();
            st.lt = 0.f;
            // the copies of this iteration (K_{j+2}, V_j) are issued without
            // branches: a tile outside [0, jend) is given an empty extent and
            // reads as zeros, into a buffer nobody reads before it is filled
            // again (K) or that is multiplied by zero terms (V).  Extents stay
            // below 2^30 bytes (host check), so these sums cannot wrap.
            const uint32_t kcopy = j + 2 < jend ? (uint32_t)((j + 2) * TILEB) : kv_bytes;
            const uint32_t vcopy = j >= 0 && j < jend ? (uint32_t)(j * TILEB) : kv_bytes;
            const auto rkt = make_rsrc(kbase + kcopy, kv_bytes - kcopy);
            const auto rvt = make_rsrc(vbase + vcopy, kv_bytes - vcopy);

            // NSLOT slots; in each: its MFMA and its share of the softmax
            // stages, then the LDS operand read of slot i + PD; one 16-byte
            // copy of the next tiles every COPY_EVERY slots
            float xs[NPAIR][2];
            u32x4_t opnd[PD + 1];
            static_for<0, PD>([&](auto I) { opnd[I.value] = slot_operand(I.value, kread, vread, ln); });
            static_for<0, NSLOT>([&](auto I) {
                constexpr int i = decltype(I)::value;
                if constexpr (i % COPY_EVERY == 1 % COPY_EVERY && i / COPY_EVERY < NCOPY) {
                    constexpr int cu = i / COPY_EVERY;
                    if constexpr (cu < LOADS) copy_part(rkt, kfill, wave, koff_c[cu], cu);
                    else copy_part(rvt, vfill, wave, voff_c[cu - LOADS], cu - LOADS);
                }
                slot_mfma(i, opnd[i % (PD + 1)], acc, snext, pk, qreg);
                if constexpr (READ_FIRST && i + PD < NSLOT) {
                    opnd[(i + PD) % (PD + 1)] = slot_operand(i + PD, kread, vread, ln);
                    __builtin_amdgcn_sched_barrier(0);
                }
                static_for<0, NPAIR>([&](auto K) {
                    constexpr int k = decltype(K)::value;
                    if constexpr (pair_slot(k) == i) stage_a(scur, k, st, c, xs[k][0], xs[k][1]);
                    if constexpr (pair_slot(k) + DB_ == i) stage_b(xs[k][0], xs[k][1]);
                    if constexpr (pair_slot(k) + DC_ == i) stage_c(pk, k, st, xs[k][0], xs[k][1]);
                });
                if constexpr (!READ_FIRST && i + PD < NSLOT)
                    opnd[(i + PD) % (PD + 1)] = slot_operand(i + PD, kread, vread, ln);
                __builtin_amdgcn_sched_barrier(0);
            });

            // the tile's sum decides the slow path (reference raised, running
            // output rescaled after this iteration's output MFMAs and before
            // the next tile's); then the tile joins the running sum
            float lt = sum_halves(st.lt);
            const bool need = lt > kTileSumLimit || lt > st.l;
            if (__builtin_amdgcn_ballot_w64(need)) {
                raise_reference(scur, pk, st, c, acc, need);
                lt = sum_halves(st.lt);
            }
            st.l += lt;
        };

        // the start is hidden from the optimiser so that it does not peel
        // the first iterations into separately allocated copies of the body
        int jstart = -1;
        asm volatile("" : "+s"(jstart));
        // iterations up to j = wend carry this wave's work (its last output
        // MFMAs run at j = wend); after that, up to jend, it only keeps up its
        // share of the workgroup's barriers and copies
        const int jlast = min(jend, wend);
#pragma clang loop unroll(disable)
        for (int j = jstart; j <= jlast; j += 2) {
            iteration(j, BoolTag<true>{});
            if (j + 1 <= jlast) iteration(j + 1, BoolTag<false>{});
        }
#pragma clang loop unroll(disable)
        for (int j = jlast + 1; j <= jend; ++j) {
            __syncthreads();
            const bool odd = j & 1;
            uint8_t* kfill = odd ? kbuf1 : kbuf0;
            uint8_t* vfill = odd ? vbuf1 : vbuf0;
            const uint32_t kcopy = j + 2 < jend ? (uint32_t)((j + 2) * TILEB) : kv_bytes;
            const uint32_t vcopy = j < jend ? (uint32_t)(j * TILEB) : kv_bytes;
            const auto rkt = make_rsrc(kbase + kcopy, kv_bytes - kcopy);
            const auto rvt = make_rsrc(vbase + vcopy, kv_bytes - vcopy);
#pragma unroll
            for (int u = 0; u < LOADS; ++u) {
                copy_part(rkt, kfill, wave, koff_c[u], u);
                copy_part(rvt, vfill, wave, voff_c[u], u);
            }
        }

        // epilogue: O = O_running / l, LSE = ln(sum exp(scale * S)) = (mc + log2 l) ln 2.
        // Lane (li, lh) holds d = 32 db + 8 jj + 4 lh + (0..3) of row q0w + li.
        const float l = st.l;
        // (a split-KV row that sees no key of its range: l = 0, O = 0, LSE = -inf)
        const float inv = SPLIT ? (l > 0.f ? 1.0f / l : 0.f) : 1.0f / l;
        // a split-KV launch writes range `split` of a [splits, B H, N] array
        const size_t out_head = SPLIT ? ((size_t)split * p.heads + hh) * N : (size_t)hh * N;
        if (OUT_F32) {
            if (qrow < N) {
                const size_t orow = (out_head + qrow) * D;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int d0 = 32 * db + 8 * jj + 4 * lh;
                        gstore((float*)out + orow + d0,
                               f32x4_t{acc[db][4 * jj + 0] * inv, acc[db][4 * jj + 1] * inv,
                                       acc[db][4 * jj + 2] * inv, acc[db][4 * jj + 3] * inv});
                    }
            }
        } else if constexpr (WAVES * 32 * ROWB <= 4 * TILEB) {
            // The 16-bit output leaves through LDS so that every store writes
            // whole rows (stored straight from the registers, each store
            // would scatter 8-byte pieces over 32 rows).  The barrier frees
            // the K / V buffers: every wave has passed its last read and its
            // copies have landed.  Each wave stages its 32 rows in its own
            // slice of them, 16-byte chunks XOR-swizzled by row against bank
            // conflicts, then stores 16 bytes per lane, CPR lanes per row.
            constexpr int CPR = ROWB / 16;              // 16-byte chunks per row
            constexpr int RPS = 64 / CPR;               // rows per store
            constexpr int SLICE = 32 * ROWB;
            static_assert(TILEB % SLICE == 0, "output staging");
            __syncthreads();
            const int sb = wave * SLICE / TILEB;
            uint8_t* const ost = (sb == 0 ? kbuf0 : sb == 1 ? kbuf1 : sb == 2 ? vbuf0 : vbuf1) + (wave * SLICE) % TILEB;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int c = 4 * db + jj;          // chunk of d = 32 db + 8 jj .. +7
                    const float o0 = acc[db][4 * jj + 0] * inv, o1 = acc[db][4 * jj + 1] * inv;
                    const float o2 = acc[db][4 * jj + 2] * inv, o3 = acc[db][4 * jj + 3] * inv;
                    *(u32x2_t*)(ost + li * ROWB + ((c ^ (li % CPR)) << 4) + 8 * lh) =
                        u32x2_t{pack2<T>(o0, o1), pack2<T>(o2, o3)};
                }
#pragma unroll
            for (int i = 0; i < 32 / RPS; ++i) {
                const int r = i * RPS + lane / CPR, c = lane % CPR;
                const u32x4_t v = *(const u32x4_t*)(ost + r * ROWB + ((c ^ (r % CPR)) << 4));
                if (q0w + r < N) gstore((uint16_t*)out + head_elems + (size_t)(q0w + r) * D + 8 * c, v);
            }
        } else {
            // (tile shapes whose K / V buffers cannot hold every wave's rows:
            // 8-byte pieces straight from the registers)
            if (qrow < N) {
                const size_t orow = head_elems + (size_t)qrow * D;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int d0 = 32 * db + 8 * jj + 4 * lh;
                        const float o0 = acc[db][4 * jj + 0] * inv, o1 = acc[db][4 * jj + 1] * inv;
                        const float o2 = acc[db][4 * jj + 2] * inv, o3 = acc[db][4 * jj + 3] * inv;
                        gstore((uint16_t*)out + orow + d0, u32x2_t{pack2<T>(o0, o1), pack2<T>(o2, o3)});
                    }
            }
        }
        if (lh == 0 && qrow < N)
            gstore(lse + out_head + qrow, SPLIT && !(l > 0.f) ? -__builtin_inff() : (st.mc + __log2f(l)) * kLn2);
        if (COUNT && tid == 0) add_tile_counts<BQ, BK, CAUSAL>(counters, qt0, jend, N);
    }
};

// ---------------------------------------------------------------------------
// Merge of split-KV partials.  Range s of a row holds the normalised output
// O_s and log-sum-exp LSE_s of that row's softmax over the range's keys
// alone.  The whole row's statistics follow from the blocked-softmax merge
// ("Flash Attention 原理", Softmax 的分块计算; the correction factor of
// "FlashAttention分块计算优化Transformer显存效率" §3.2): with
// LSE = ln sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s.
// A thread merges 8 consecutive columns of one row.
// ---------------------------------------------------------------------------
template <class T, int D>
__global__ void __launch_bounds__(256) split_merge_kernel(const float* opart, const float* lpart, void* o,
                                                          float* lse, int rows, int splits) {
    // a thread merges 8 consecutive columns of one row: D / 8 threads per
    // row, 16-byte loads of the fp32 partials and one 16-byte store
    constexpr int TPR = D / 8;                      // threads per row
    const int t = blockIdx.x * 256 + threadIdx.x;
    const int row = t / TPR, c0 = (t % TPR) * 8;
    if (row >= rows) return;                        // no barrier follows
    float m = -__builtin_inff();
    for (int s = 0; s < splits; ++s) m = fmaxf(m, lpart[(size_t)s * rows + row]);
    float den = 0.f;
    for (int s = 0; s < splits; ++s) den += expf(lpart[(size_t)s * rows + row] - m);
    const float total = m + logf(den);
    float acc[8] = {};
    for (int s = 0; s < splits; ++s) {
        const float w = expf(lpart[(size_t)s * rows + row] - total);
        const f32x4_t* src = (const f32x4_t*)(opart + ((size_t)s * rows + row) * D + c0);
        const f32x4_t a = src[0], b = src[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[e] += w * a[e];
            acc[4 + e] += w * b[e];
        }
    }
    if constexpr (__is_same(T, float)) {   // fp32 output
        gstore((float*)o + (size_t)row * D + c0, f32x4_t{acc[0], acc[1], acc[2], acc[3]});
        gstore((float*)o + (size_t)row * D + c0 + 4, f32x4_t{acc[4], acc[5], acc[6], acc[7]});
    } else {
        gstore((uint16_t*)o + (size_t)row * D + c0,
               u32x4_t{pack2<T>(acc[0], acc[1]), pack2<T>(acc[2], acc[3]), pack2<T>(acc[4], acc[5]),
                       pack2<T>(acc[6], acc[7])});
    }
    if (c0 == 0) gstore(lse + row, total);
}

// ---------------------------------------------------------------------------
// Persistent 16-bit kernel (16-bit output, no counters).
//
// One workgroup per workgroup slot of the device (one per CU without a
// mask) stays resident and takes the query tiles b, b + G, b + 2 G, ... of
// the logical order above (G workgroups; with G a multiple of 8 every tile
// of a workgroup lies on its XCD's range).  Its waves run
// the key loops of those tiles back to back as one stream of key tiles, so
// the software pipeline of Fwd16 neither drains nor refills between query
// tiles: while the output MFMAs finish a tile's last key tile, the score
// MFMAs already run on the next tile's first.  At the iteration whose
// softmax takes key tile j of a query tile (nk key tiles per query tile):
//   j = 0       the previous query tile's LSE is stored and the softmax
//               state restarts; the first-key slow path leaves the
//               accumulators alone (they still hold that tile's output);
//   j = 1       the previous tile's output, final after the output MFMAs of
//               iteration j = 0, leaves through LDS (right after the barrier,
//               before any copy of the iteration is issued), and the
//               accumulators clear;
//   j = 2       the next tile's Q rows are copied HBM -> LDS (direct-to-LDS
//               loads into the wave's own staging slice);
//   j = nk - 1  the next tile's Q^T operands are read from that slice: the
//               score MFMAs of this iteration start the next tile.
// Without a mask the host uses it for nk >= 4, where these are four
// different iterations.
//
// Causal variant (WIDE, d = 128): a query tile costs its own number of key
// tiles, so a workgroup takes pairs of query tiles (i, T - 1 - i) of a head,
// whose costs add up to the same for every pair.  With eight waves (256-row
// query tiles, one workgroup per CU) every query tile has at least four key
// tiles, so the transitions above apply unchanged, and the diagonal's masks
// fall on the last four key tiles of a query tile.
// ---------------------------------------------------------------------------
template <class T, int D, bool CAUSAL = false, bool WIDE = false>
struct Fwd16P {
    using Bs = Fwd16<T, D, CAUSAL, false, false, 8>;
    static constexpr int WAVES = Bs::WAVES, BQ = Bs::BQ, OCC = Bs::OCC, NT = Bs::NT, BK = Bs::BK;
    static constexpr int RESIDENT = Bs::RESIDENT;
    static constexpr int ROWB = Bs::ROWB, TILEB = Bs::TILEB, NS = Bs::NS, NDB = Bs::NDB, NMB = Bs::NMB;
    static constexpr int NKS = Bs::NKS, NSLOT = Bs::NSLOT, NPAIR = Bs::NPAIR, PD = Bs::PD, LOADS = Bs::LOADS;
    static constexpr int DB_ = Bs::DB_, DC_ = Bs::DC_, COPY_EVERY = Bs::COPY_EVERY, NCOPY = Bs::NCOPY;
    static constexpr bool READ_FIRST = Bs::READ_FIRST;
    static constexpr int SLICE = 32 * ROWB;          // one wave's Q / O staging bytes
    static constexpr int QLOADS = SLICE / 1024;      // 16-byte copies per lane of a wave's Q rows
    static constexpr int MIN_KEY_TILES = 4;
    static constexpr int QCOPY_AT = 2;               // key tile at which the next Q rows are copied
    static constexpr int STEADY_LO = 3;              // plain iterations: STEADY_LO <= j <= nk - 1 - TAIL
    // key tiles at the end of a query tile that are never plain: the K copy
    // of j + 2 crosses into the next tile from j = nk - 2 on, and under the
    // mask the diagonal covers the last BQ / BK key tiles
    static constexpr int TAIL = CAUSAL ? BQ / BK : 2;
    static constexpr int CPR = ROWB / 16;            // 16-byte chunks per row
    static constexpr int RPS = 64 / CPR;             // rows per 16-byte store
    static_assert(SLICE % 1024 == 0 && RESIDENT == 1, "persistent shape");
    static_assert(WIDE == CAUSAL && WAVES == 8, "the causal kernel has 256-row query tiles");
    static_assert(!CAUSAL || BQ / BK > 2, "the diagonal's key tiles are never plain iterations");
    static_assert(4 * TILEB + WAVES * SLICE <= 160 * 1024, "LDS per CU");

    // The lane index, opaque to the optimiser: addresses derived from it in a
    // once-per-tile block are computed there, not hoisted out of the key loop
    // into registers that would stay live through it.
    static __device__ __forceinline__ int opaque_lane(int lane) {
        asm volatile("" : "+v"(lane));
        return lane;
    }

    struct TileInfo {
        size_t hoff;        // byte offset of the head in Q, K, V and O
        int hh;             // head (batch * H + h)
        int qt0;            // first query row
        int nk;             // key tiles of the query tile
    };

    // Output of one query tile: acc / l rounded to 16 bits, staged in the
    // wave's slice (16-byte chunks XOR-swizzled by row), stored as whole rows.
    // Inside the key loop every other register is live, so the pieces go one
    // at a time (scheduling barriers keep the compiler from computing them
    // all first).
    static __device__ __forceinline__ void store_output(const f32x16_t* acc, float inv, uint8_t* ost, void* out,
                                                        const TileInfo& t, int wave, int lane, int N) {
        lane = opaque_lane(lane);
        const int li = lane & 31, lh = lane >> 5;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int c = 4 * db + jj;
                const float o0 = acc[db][4 * jj + 0] * inv, o1 = acc[db][4 * jj + 1] * inv;
                const float o2 = acc[db][4 * jj + 2] * inv, o3 = acc[db][4 * jj + 3] * inv;
                *(u32x2_t*)(ost + li * ROWB + ((c ^ (li % CPR)) << 4) + 8 * lh) =
                    u32x2_t{pack2<T>(o0, o1), pack2<T>(o2, o3)};
                __builtin_amdgcn_sched_barrier(0);
            }
        const int q0w = t.qt0 + wave * 32;
        uint8_t* const obase = (uint8_t*)out + t.hoff;
#pragma unroll
        for (int i = 0; i < 32 / RPS; ++i) {
            const int r = i * RPS + lane / CPR, c = lane % CPR;
            const u32x4_t v = *(const u32x4_t*)(ost + r * ROWB + ((c ^ (r % CPR)) << 4));
            if (q0w + r < N) gstore(obase + (size_t)(q0w + r) * ROWB + 16 * c, v);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    static __device__ void run(const FwdParams& p) { run_impl<false>(p); }

    // COUNT: the instrumented instance (Fwd16PCount) adds the tile counts of
    // the (query tile, key tile) pairs its iterations process to p.counters
    template <bool COUNT>
    static __device__ void run_impl(const FwdParams& p) {
        __shared__ __attribute__((aligned(1024))) uint8_t kbuf0[TILEB];
        __shared__ __attribute__((aligned(1024))) uint8_t kbuf1[TILEB];
        __shared__ __attribute__((aligned(1024))) uint8_t vbuf0[TILEB];
        __shared__ __attribute__((aligned(1024))) uint8_t vbuf1[TILEB];
        // (less aligned than the K / V buffers, which the allocator then
        // places first: their operand reads keep addresses below 64 KiB,
        // which the 16-bit offset field of an LDS instruction can reach)
        __shared__ __attribute__((aligned(256))) uint8_t qbuf[WAVES * SLICE];
        const int tid = threadIdx.x;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int lane = tid & 63;
        const int li = lane & 31, lh = lane >> 5;
        const int N = p.N;
        // every kernel argument in SGPRs before the first direct-to-LDS copy
        void* const out = pin_s(p.o);
        float* const lse = pin_s(p.lse);
        const float c = pin_s(p.c);
        const uint32_t qsign = pin_s(p.qsign);
        const uint8_t* const qptr = (const uint8_t*)pin_s(p.q);
        const uint8_t* const kptr = (const uint8_t*)pin_s(p.k);
        const uint8_t* const vptr = (const uint8_t*)pin_s(p.v);
        const int tiles_q = pin_s(p.tiles_q);
        const int total = pin_s(p.total);
        unsigned long long* const counters = COUNT ? pin_s(p.counters) : nullptr;
        uint32_t n_iter = 0;   // iterations that processed a (query tile, key tile) pair

        const int G = gridDim.x, b = blockIdx.x;
        // work units: query tiles, or (causal) pairs of query tiles; b < units
        const int units = CAUSAL ? total / 2 : total;
        const int ntiles = (CAUSAL ? 2 : 1) * ((units - b + G - 1) / G);
        const int nk_all = (N + BK - 1) / BK;           // >= MIN_KEY_TILES
        const uint32_t head_bytes = (uint32_t)N * ROWB;
        uint8_t* const qslice = qbuf + wave * SLICE;

        auto decode = [&](int k) {
            k = min(k, ntiles - 1);
            int hh, qi;
            if (CAUSAL) {
                const int half = tiles_q / 2;
                const int L = xcd_remap(b + (k >> 1) * G, units);
                hh = L / half;
                const int i = L - hh * half;
                qi = (k & 1) ? i : tiles_q - 1 - i;
            } else {
                const int L = xcd_remap(b + k * G, units);
                hh = L / tiles_q;
                qi = L - hh * tiles_q;
            }
            const int qt0 = qi * BQ;
            const int nkt = CAUSAL ? (min(qt0 + BQ, N) - 1) / BK + 1 : nk_all;
            return TileInfo{(size_t)hh * head_bytes, hh, qt0, nkt};
        };
        int gend = 0;                                   // key tiles of this workgroup
        if (CAUSAL) {
            for (int k = 0; k < ntiles; ++k) gend += decode(k).nk;
        } else {
            gend = ntiles * nk_all;
        }
        asm volatile("" : "+s"(gend));
        TileInfo cur = decode(0), nxt = decode(1), prv = cur;

        // zero fill before the first copy (see Fwd16)
#pragma unroll
        for (int i = tid; i < TILEB / 16; i += NT) {
            ((u32x4_t*)vbuf0)[i] = u32x4_t{0, 0, 0, 0};
            ((u32x4_t*)vbuf1)[i] = u32x4_t{0, 0, 0, 0};
            ((u32x4_t*)kbuf1)[i] = u32x4_t{0, 0, 0, 0};
        }

        // Q^T operand of the first tile straight from HBM
        u32x4_t qreg[NS];
        {
            const auto rq = make_rsrc(qptr + cur.hoff, head_bytes);
            const int qrow = cur.qt0 + wave * 32 + li;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                qreg[s] = buf_load16(rq, (uint32_t)(qrow * D + 16 * s + 8 * lh) * 2);
                qreg[s] ^= qsign;
            }
        }

        typename Bs::Lane ln;
        {
            const int prow = Bs::perm_row(li);
            const int ks_sw = Bs::fk(prow);
#pragma unroll
            for (int ks = 0; ks < NS; ++ks) ln.koff[ks] = prow * ROWB + (((2 * ks + lh) ^ ks_sw) << 4);
            const int Gq = lane >> 4, sq = lane & 15;
            const int fvq = D == 128 ? ((sq >> 2) & 3) : ((sq >> 3) & 1);
            const int y = 2 * (Gq & 1) + ((sq & 3) >> 1);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                ln.voff[db] = (8 * lh + (sq >> 2)) * ROWB + ((4 * (db ^ fvq) + y) << 4) + 8 * (sq & 1);
        }

        f32x16_t acc[NDB];
        f32x16_t s0[NMB], s1[NMB];
        u32x4_t pk[NKS];
        typename Bs::Soft st;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] = f32x16_t{};
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) s0[mb] = s1[mb] = f32x16_t{};
#pragma unroll
        for (int kt = 0; kt < NKS; ++kt) pk[kt] = u32x4_t{0, 0, 0, 0};
        st.mc = -__FLT_MAX__;
        st.l = st.lt = 0.f;
        float inv_prev = 0.f;

        const uint32_t ksrc = Bs::template copy_offset<true>(wave, lane);
        const uint32_t vsrc = Bs::template copy_offset<false>(wave, lane);
        uint32_t koff_c[LOADS], voff_c[LOADS];
#pragma unroll
        for (int u = 0; u < LOADS; ++u) {
            koff_c[u] = ksrc + (uint32_t)(u * WAVES * 1024);
            voff_c[u] = vsrc + (uint32_t)(u * WAVES * 1024);
        }

        {   // K_0 of the first tile into kbuf0
            const auto rk0 = make_rsrc(kptr + cur.hoff, head_bytes);
#pragma unroll
            for (int u = 0; u < LOADS; ++u) Bs::copy_part(rk0, kbuf0, wave, koff_c[u], u);
        }

        // position of the softmax stream: key tile j0 of this workgroup's
        // query tile k0 (j0 = -1 before the first; j0 = nk until the wrap)
        int k0 = 0, j0 = -1;
        // iterations with STEADY_LO <= j0 <= nk - 1 - TAIL are plain: one
        // range check, the copy sources advance by a tile; every other one
        // recomputes its state in one block (and applies the masks, so the
        // last TAIL key tiles -- the K copy crossing into the next tile, and
        // under the mask the diagonal's tiles -- are never plain)
        auto steady_count = [&](int nkt) {
            return nkt > STEADY_LO + TAIL ? (uint32_t)(nkt - STEADY_LO - TAIL) : 0u;
        };
        uint32_t nk_s = steady_count(cur.nk);
        const uint8_t* kc_ptr = kptr;      // K copy of this iteration (key tile g + 2)
        const uint8_t* vc_ptr = vptr;      // V copy (key tile g)
        uint32_t kc_ext = 0, vc_ext = 0;
        bool sm_on = false;                // this wave has rows in the softmax tile

        auto iteration = [&](const int g, auto odd_tag) __attribute__((always_inline)) {
            constexpr bool ODD = decltype(odd_tag)::value;
            uint8_t* kread = ODD ? kbuf0 : kbuf1;
            uint8_t* kfill = ODD ? kbuf1 : kbuf0;
            uint8_t* vread = ODD ? vbuf0 : vbuf1;
            uint8_t* vfill = ODD ? vbuf1 : vbuf0;
            f32x16_t* scur = ODD ? s1 : s0;
            f32x16_t* snext = ODD ? s0 : s1;

            __syncthreads();   // this wave's copies done (vmcnt 0), and everyone's

            if ((uint32_t)(j0 - STEADY_LO) >= nk_s) {
                if (j0 == cur.nk) {
                    j0 = 0;
                    ++k0;
                }
                if (j0 == 1 && k0 >= 1) {
                    // the previous tile's output (no copy of this wave in flight)
                    store_output(acc, inv_prev, qslice, out, prv, wave, lane, N);
#pragma unroll
                    for (int db = 0; db < NDB; ++db) acc[db] = f32x16_t{};
                }
                if (j0 == 0 && k0 >= 1) {
                    // the tile k0 - 1 is complete: its LSE, and a fresh softmax state
                    const int row = cur.qt0 + wave * 32 + li;
                    if (lh == 0 && row < N) gstore(lse + (size_t)cur.hh * N + row, (st.mc + __log2f(st.l)) * kLn2);
                    inv_prev = 1.0f / st.l;
                    st.mc = -__FLT_MAX__;
                    st.l = 0.f;
                    prv = cur;
                    cur = nxt;
                    nxt = decode(k0 + 1);
                    nk_s = steady_count(cur.nk);
                }
                if (j0 == QCOPY_AT && k0 + 1 < ntiles) {
                    // the next tile's Q rows into this wave's slice, chunks
                    // XOR-swizzled by row as the operand reads below expect
                    const uint32_t r0 = (uint32_t)(nxt.qt0 + wave * 32) * ROWB;
                    const uint32_t ext = __builtin_amdgcn_readfirstlane(r0 < head_bytes ? head_bytes - r0 : 0u);
                    const auto rq = make_rsrc(qptr + nxt.hoff + r0, ext);
                    const int ol = opaque_lane(lane);
#pragma unroll
                    for (int u = 0; u < QLOADS; ++u) {
                        const int o = u * 1024 + ol * 16, r = o / ROWB;
                        const uint32_t src = (uint32_t)(r * ROWB + ((((o % ROWB) >> 4) ^ Bs::fk(r)) << 4));
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            rq, (__attribute__((address_space(3))) void*)(qslice + u * 1024), 16, src, 0, 0, 0);
                    }
                }
                if (j0 == cur.nk - 1 && k0 + 1 < ntiles) {
                    // the score MFMAs of this iteration start the next tile
                    const int ol = opaque_lane(lane), oli = ol & 31, olh = ol >> 5;
                    const uint8_t* qs = qslice + oli * ROWB;
#pragma unroll
                    for (int s = 0; s < NS; ++s) {
                        qreg[s] = *(const u32x4_t*)(qs + (((2 * s + olh) ^ Bs::fk(oli)) << 4));
                        qreg[s] ^= qsign;
                    }
                }
                const int q0w = cur.qt0 + wave * 32;
                sm_on = j0 >= 0 && k0 < ntiles && q0w < N;
                const int kk0 = j0 * BK;
                if (sm_on && ((CAUSAL && kk0 + BK - 1 > q0w) || kk0 + BK > N)) {
                    // the diagonal and the ragged last key tile
                    int lim = N - 1 - kk0 - 8 * lh;
                    if (CAUSAL) lim = min(lim, q0w + li - kk0 - 8 * lh);
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int kk = 32 * mb + 16 * (r >> 3) + (r & 7);
                            scur[mb][r] = kk > lim ? -__builtin_inff() : scur[mb][r];
                        }
                }
                // copy sources: K of key tile g + 2 and V of key tile g of the
                // stream (empty extents outside it)
                const bool kin = j0 + 2 < cur.nk;
                const uint32_t kcopy = g + 2 < gend ? (uint32_t)((kin ? j0 + 2 : j0 + 2 - cur.nk) * TILEB) : head_bytes;
                const uint32_t vcopy = j0 >= 0 && g < gend ? (uint32_t)(j0 * TILEB) : head_bytes;
                kc_ptr = kptr + (kin ? cur.hoff : nxt.hoff) + kcopy;
                kc_ext = head_bytes - kcopy;
                vc_ptr = vptr + cur.hoff + vcopy;
                vc_ext = head_bytes - vcopy;
            }
            if constexpr (COUNT) {
                // this iteration's softmax runs on the pair (query tile k0, key tile j0)
                if (j0 >= 0 && j0 < cur.nk && k0 < ntiles) ++n_iter;
            }
            st.meff = sm_on ? st.mc : __builtin_inff();
            st.lt = 0.f;
            const auto rkt = make_rsrc(kc_ptr, kc_ext);
            const auto rvt = make_rsrc(vc_ptr, vc_ext);

            float xs[NPAIR][2];
            u32x4_t opnd[PD + 1];
            static_for<0, PD>([&](auto I) { opnd[I.value] = Bs::slot_operand(I.value, kread, vread, ln); });
            static_for<0, NSLOT>([&](auto I) {
                constexpr int i = decltype(I)::value;
                if constexpr (i % COPY_EVERY == 1 % COPY_EVERY && i / COPY_EVERY < NCOPY) {
                    constexpr int cu = i / COPY_EVERY;
                    if constexpr (cu < LOADS) Bs::copy_part(rkt, kfill, wave, koff_c[cu], cu);
                    else Bs::copy_part(rvt, vfill, wave, voff_c[cu - LOADS], cu - LOADS);
                }
                Bs::slot_mfma(i, opnd[i % (PD + 1)], acc, snext, pk, qreg);
                if constexpr (READ_FIRST && i + PD < NSLOT) {
                    opnd[(i + PD) % (PD + 1)] = Bs::slot_operand(i + PD, kread, vread, ln);
                    __builtin_amdgcn_sched_barrier(0);
                }
                static_for<0, NPAIR>([&](auto K) {
                    constexpr int k = decltype(K)::value;
                    if constexpr (Bs::pair_slot(k) == i) Bs::stage_a(scur, k, st, c, xs[k][0], xs[k][1]);
                    if constexpr (Bs::pair_slot(k) + DB_ == i) Bs::stage_b(xs[k][0], xs[k][1]);
                    if constexpr (Bs::pair_slot(k) + DC_ == i) Bs::stage_c(pk, k, st, xs[k][0], xs[k][1]);
                });
                if constexpr (!READ_FIRST && i + PD < NSLOT)
                    opnd[(i + PD) % (PD + 1)] = Bs::slot_operand(i + PD, kread, vread, ln);
                __builtin_amdgcn_sched_barrier(0);
            });

            float lt = sum_halves(st.lt);
            const bool need = lt > Bs::kTileSumLimit || lt > st.l;
            if (__builtin_amdgcn_ballot_w64(need)) {
                Bs::raise_reference(scur, pk, st, c, acc, need, j0 == 0);
                lt = sum_halves(st.lt);
            }
            st.l += lt;
            // the next iteration's copy sources if it is a plain one (a
            // recomputing one overwrites them; extents that hit zero here are
            // only ever followed by recomputing iterations)
            kc_ptr += TILEB;
            kc_ext -= TILEB;
            vc_ptr += TILEB;
            vc_ext -= TILEB;
            ++j0;
        };

        int gstart = -1;
        asm volatile("" : "+s"(gstart));
#pragma clang loop unroll(disable)
        for (int g = gstart; g <= gend; g += 2) {
            iteration(g, BoolTag<true>{});
            if (g + 1 <= gend) iteration(g + 1, BoolTag<false>{});
        }

        // the last tile's output (its LSE was stored at the iteration g = gend)
        __syncthreads();
        store_output(acc, inv_prev, qslice, out, prv, wave, lane, N);
        if constexpr (COUNT) {
            // The pairs of the query tiles this workgroup processed, classed
            // as in add_tile_counts: key tiles [0, nk) of each were visited,
            // the rest of the head's key tiles skipped.  The computed count is
            // the number of iterations that visited a pair; a decomposition
            // that disagrees with the loop (the sum of nk over the tiles)
            // shows as a computed count different from the classes' sum.
            if (tid == 0) {
                uint32_t full = 0, masked = 0, ragged = 0, skipped = 0;
                for (int k = 0; k < ntiles; ++k) {
                    const TileInfo t = decode(k);
                    skipped += (uint32_t)(nk_all - t.nk);
                    for (int j = 0; j < t.nk; ++j) {
                        const int kk = j * BK;
                        if (CAUSAL && kk + BK - 1 > t.qt0) ++masked;
                        else if (kk + BK > N) ++ragged;
                        else ++full;
                    }
                }
                atomicAdd(counters + 0, (unsigned long long)n_iter);
                atomicAdd(counters + 1, (unsigned long long)full);
                atomicAdd(counters + 2, (unsigned long long)masked);
                atomicAdd(counters + 3, (unsigned long long)ragged);
                atomicAdd(counters + 4, (unsigned long long)skipped);
            }
        }
    }
};

// The instrumented persistent kernel: the same code, plus the tile counts of
// the pairs its iterations process (p.counters, as in Fwd16 with COUNT).
template <class T, int D, bool CAUSAL = false, bool WIDE = false>
struct Fwd16PCount : Fwd16P<T, D, CAUSAL, WIDE> {
    static __device__ void run(const FwdParams& p) { Fwd16P<T, D, CAUSAL, WIDE>::template run_impl<true>(p); }
};

// ---------------------------------------------------------------------------
// fp32 kernel: fp32 MFMA (v_mfma_f32_32x32x2_f32), 64 x 64 tiles
// ---------------------------------------------------------------------------

// SPLIT: a split-KV launch (see Fwd16): one query tile over one range of
// p.split_len keys, the range's partial output and log-sum-exp written to
// range `split` of the fp32 work arrays; a row that sees no key of its range
// leaves O = 0, LSE = -inf.
template <int D, bool CAUSAL, bool COUNT, bool SPLIT = false>
struct Fwd32 {
    static constexpr int BQ = 64;                  // 2 waves x 32 query rows
    static constexpr int WAVES = 2;
    static constexpr int OCC = 1;
    static constexpr int RESIDENT = 4 * OCC / WAVES;   // workgroups per CU
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

        TileId t;
        int split = 0;
        if constexpr (SPLIT && CAUSAL) {
            // (query tile, head, range), longest tiles first across the XCDs
            const int per_rank = p.heads * p.splits;
            const int rank = blockIdx.x / per_rank, rem = blockIdx.x - rank * per_rank;
            t.qi = p.tiles_q - 1 - rank;
            t.hh = rem / p.splits;
            split = rem - t.hh * p.splits;
        } else if constexpr (SPLIT) {
            const int L = xcd_remap(blockIdx.x, p.total * p.splits);
            const int per_head = p.tiles_q * p.splits;
            t.hh = L / per_head;
            const int rem = L - t.hh * per_head;
            t.qi = rem / p.splits;
            split = rem - t.qi * p.splits;
        } else {
            t = tile_of<CAUSAL>(blockIdx.x, p);
        }
        const int hh = t.hh;
        const int qt0 = t.qi * BQ;
        const int q0w = qt0 + wave * 32;
        const int qrow = q0w + li;

        const size_t head_elems = (size_t)hh * N * D;
        const uint32_t head_bytes = (uint32_t)N * D * 4;
        const auto rq = make_rsrc((const uint8_t*)p.q + head_elems * 4, head_bytes);
        // the keys this workgroup visits: the head's, or one range of them
        const int kfirst = SPLIT ? split * p.split_len : 0;
        const int NK = SPLIT ? min(p.split_len, N - kfirst) : N;
        const uint32_t kv_bytes = (uint32_t)NK * D * 4;
        const auto rk = make_rsrc((const uint8_t*)p.k + (head_elems + (size_t)kfirst * D) * 4, kv_bytes);
        const auto rv = make_rsrc((const uint8_t*)p.v + (head_elems + (size_t)kfirst * D) * 4, kv_bytes);

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

        const int nk = (NK + BK - 1) / BK;
        int jend;
        if constexpr (SPLIT && CAUSAL) {
            const int kmax = min(qt0 + BQ, N) - 1 - kfirst;
            jend = kmax < 0 ? 0 : min(nk, kmax / BK + 1);
        } else {
            jend = CAUSAL ? (min(qt0 + BQ, N) - 1) / BK + 1 : nk;
        }

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
            const bool active = (!CAUSAL || kfirst + k0 <= q0w + 31) && q0w < N;
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
                const bool need_mask = (CAUSAL && kfirst + k0 + BK - 1 > q0w) || (k0 + BK > NK);
                if (need_mask) {
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int key = k0 + 32 * mb + 16 * (r >> 3) + 8 * lh + (r & 7);
                            if ((CAUSAL && kfirst + key > qrow) || key >= NK) s[mb][r] = -__builtin_inff();
                        }
                }
                float mx = -__builtin_inff();
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[mb][r]);
                mx = max_halves(mx);
                const float mnew = __builtin_fmaxf(m, mx);
                float alpha = __builtin_amdgcn_exp2f((m - mnew) * c);
                float mc = mnew * c;
                if constexpr (SPLIT) {
                    // a row with no visible key so far: correction 1, terms 0
                    const bool none = mnew == -__builtin_inff();
                    alpha = none ? 1.0f : alpha;
                    mc = none ? 0.f : mc;
                }
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
        // a split-KV launch writes range `split` of a [splits, B H, N] array
        const size_t out_head = SPLIT ? ((size_t)split * p.heads + hh) * N : (size_t)hh * N;
        if (q0w < N && qrow < N) {
            const float inv = SPLIT ? (lt > 0.f ? 1.0f / lt : 0.f) : 1.0f / lt;
            const size_t orow = (out_head + qrow) * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int d0 = 32 * db + 8 * jj + 4 * lh;
                    *(f32x4_t*)((float*)p.o + orow + d0) =
                        f32x4_t{acc[db][4 * jj] * inv, acc[db][4 * jj + 1] * inv,
                                acc[db][4 * jj + 2] * inv, acc[db][4 * jj + 3] * inv};
                }
            if (lh == 0)
                p.lse[out_head + qrow] = SPLIT && !(lt > 0.f) ? -__builtin_inff() : (m * c + __log2f(lt)) * kLn2;
        }
        if (COUNT && tid == 0) add_tile_counts<BQ, BK, CAUSAL>(p.counters, qt0, jend, N);
    }
};

template <class K>
__global__ void __launch_bounds__(K::NT) __attribute__((amdgpu_waves_per_eu(K::OCC, K::OCC))) fwd_kernel(FwdParams p) {
    K::run(p);
}

}  // namespace fa
