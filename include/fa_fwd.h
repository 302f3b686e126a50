/*
 * fa_fwd.h -- C ABI of the MI355X (gfx950) FlashAttention forward library.
 *
 * The operation (from "FlashAttention分块计算优化Transformer显存效率",
 * §1.1 standard vs. tiled attention, §2.2 causal masking, §3.2 online
 * softmax; and "Flash Attention 原理", blocked softmax and the statistics
 * kept for a recomputing backward pass):
 *
 *   for every batch b and head h, with Q, K, V the N x d matrices of that head
 *   (rows are tokens):
 *     S      = scale * Q K^T                           (N x N, never stored)
 *     S[i,j] = -inf where j > i                        (causal only; the
 *                                                        diagonal is visible)
 *     P      = row-softmax(S)                          (never stored)
 *     O      = P V                                     (N x d, stored)
 *     LSE[i] = ln sum_j exp(S[i,j])                    (stored, fp32)
 *
 * computed tile by tile with a running row maximum and running row sum that
 * rescale a partial output; key tiles entirely above the diagonal are not
 * loaded under the causal mask.
 *
 * Layout.  q, k, v and o are dense row-major [B, H, N, d] device arrays (each
 * head is an N x d matrix with contiguous rows, element stride 1, row stride
 * d).  lse is a dense [B, H, N] fp32 device array.  No other strides are
 * accepted: a caller holding [B, N, H, d] makes it contiguous first.
 *
 * Element types.  fa_fwd_bf16 / fa_fwd_f16 / fa_fwd_f32 read bfloat16 /
 * IEEE half / fp32 inputs and write o in the same type.  The products Q K^T
 * and P V run on the matrix cores with fp32 accumulation; the softmax runs in
 * fp32; P is rounded (to nearest even) to the input type before P V, and o
 * is rounded to nearest even on store.  fp32 inputs use fp32 matrix-core
 * arithmetic throughout.
 *
 * Sizes.  B, H, N, d > 0.  d must be 64 or 128.  N * d * elem_size must be
 * below 2^31 bytes per head, and B * H * ceil(N / tile_q) below 2^31.
 *
 * Ownership and concurrency.  The caller allocates every buffer.  The library
 * allocates no device memory, keeps no per-call state and may be called from
 * several host threads.  Work is enqueued on `stream` (a hipStream_t passed
 * as an opaque pointer; NULL is the default stream) and the call returns
 * without synchronising.  q, k and v may alias one another; o and lse must
 * not overlap any input or each other.
 *
 * Errors.  Every argument check runs before any HIP call and returns
 * synchronously; nothing is enqueued when a check fails.  The library never
 * prints and never throws.  A fault inside a kernel surfaces at the caller's
 * next synchronisation.  Non-finite input values propagate to the outputs of
 * the rows that see them; they are not masked.
 */
#ifndef FA_FWD_H
#define FA_FWD_H

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
typedef enum {
    FA_OK = 0,
    FA_ERR_INVALID = 1,      /* B, H, N or d <= 0 (sizes must be positive),
                                a NULL pointer, causal not 0 or 1, scale not
                                finite, o / lse overlapping an input or each
                                other, unknown out_dtype                     */
    FA_ERR_UNSUPPORTED = 2,  /* d not 64 or 128, unknown dtype, tile shape not
                                built, sizes beyond the limits above, device
                                not gfx950                                    */
    FA_ERR_HIP = 3,          /* a HIP runtime call (device query or kernel
                                launch) failed                               */
    FA_ERR_SCRATCH = 4       /* the problem needs more work memory than the
                                fixed scratch array of a no-allocation entry
                                point holds (fa_bwd.h, fa_bwd_noalloc)       */
} fa_status;

/* Element types of q, k, v (and of o unless out_dtype says fp32). */
typedef enum { FA_DTYPE_F32 = 0, FA_DTYPE_F16 = 1, FA_DTYPE_BF16 = 2 } fa_dtype;

/* Indices into the optional tile-counter array of fa_fwd_ex. */
enum {
    FA_COUNT_COMPUTED = 0,      /* (query tile, key tile) pairs processed     */
    FA_COUNT_FULL = 1,          /* ... of which unmasked and full length      */
    FA_COUNT_CAUSAL_MASKED = 2, /* ... of which reach past the diagonal       */
    FA_COUNT_RAGGED = 3,        /* ... of which are the short last key tile   */
    FA_COUNT_SKIPPED = 4,       /* pairs above the diagonal, never loaded     */
    FA_NUM_COUNTERS = 5
};

/*
 * The forward pass, one entry point per element type, with the parameter list
 * of the problem statement:
 *   q, k, v  device pointers to [B, H, N, d] inputs (read only)
 *   o        device pointer to the [B, H, N, d] output, same element type
 *   lse      device pointer to the [B, H, N] fp32 log-sum-exp output
 *   B, H, N, d  batch, heads, sequence length, head dimension
 *   scale    multiplies Q K^T (1/sqrt(d) in the pages); any finite value
 *   causal   0: every key visible; 1: key j visible to query i iff j <= i
 *   stream   hipStream_t (opaque), or NULL
 * Returns an fa_status.
 */
int fa_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int H, int N, int d, float scale, int causal, void* stream);
int fa_fwd_f16(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, float scale, int causal, void* stream);
int fa_fwd_f32(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, float scale, int causal, void* stream);

/* The same twelve parameters followed by the element type (an fa_dtype). */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, void* stream,
           int dtype);

/*
 * Extended form for validation and measurement.  Same semantics, plus:
 *   out_dtype  0: o has the input element type; 1: o is fp32 (the output is
 *              then not rounded to 16 bits -- used to check the kernel's
 *              arithmetic separately from the final rounding)
 *   tile_q, tile_k  0 selects the library default (see fa_fwd_tile_shape);
 *              otherwise the shape must be one that was built: the default,
 *              or for bf16, d = 128, no mask and 16-bit output any of
 *              tile_q in {64, 128, 256} x tile_k in {32, 64, 128} (a tile-size
 *              sweep after "FlashAttention Memory Model" Q3, the tile-size
 *              trade-off; a launch that names one of these shapes, the
 *              default included, uses the per-tile kernel of that shape).
 *              FA_ERR_UNSUPPORTED otherwise.
 *   counters   NULL for the plain kernel; otherwise a device array of
 *              FA_NUM_COUNTERS unsigned 64-bit integers to which the launch
 *              ADDS its tile counts (indices above), in the tile of
 *              fa_fwd_launch_tile: each (query tile, key tile) pair the
 *              kernel's loop processes is counted and classed, and the
 *              pairs of each processed query tile that the loop does not
 *              visit are counted as skipped.  The caller zeroes it.  A
 *              separately compiled instrumented instance of the kernel the
 *              plain launch runs is used; the plain kernel carries no
 *              counting code.
 */
typedef struct {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, H, N, d;
    float scale;
    int causal;
    void* stream;
    int dtype;
    int out_dtype;
    int tile_q, tile_k;
    unsigned long long* counters;
} fa_fwd_args;

int fa_fwd_ex(const fa_fwd_args* args);

/*
 * Split-KV forward: the keys of every head are cut into
 * `splits` ranges of whole 64-key tiles (fewer when N has fewer key tiles),
 * each (query tile, key range) runs as its own workgroup and writes the
 * partial output and log-sum-exp of its range's softmax in fp32, and a
 * second kernel merges the ranges of every row with the blocked-softmax rule
 * of "Flash Attention 原理" (Softmax 的分块计算) -- the correction factor of
 * §3.2 of "FlashAttention分块计算优化Transformer显存效率" applied once per
 * range: LSE = ln sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s.  Under
 * the causal mask a range with no key visible to a row contributes O = 0,
 * LSE = -inf (weight 0).  Same result as fa_fwd up to rounding; it fills the
 * device when B * H * N is too small for one workgroup per query tile to do
 * so, and under the mask it cuts the longest rows into pieces.
 *   o, lse     outputs, as for fa_fwd
 *   o_part     device work array of splits * B * H * N * d fp32
 *   lse_part   device work array of splits * B * H * N fp32
 *   causal     as for fa_fwd
 *   splits     key ranges requested, >= 1
 *   dtype      FA_DTYPE_BF16, FA_DTYPE_F16 or FA_DTYPE_F32 (fp32: 64-row query
 *              tiles on the fp32 matrix cores, fp32 output)
 * The caller allocates the work arrays; they must not overlap any input,
 * output or each other (FA_ERR_INVALID), nor may splits be < 1; other checks
 * as for fa_fwd.
 */
int fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                 float* o_part, float* lse_part, int B, int H, int N, int d,
                 float scale, int causal, int splits, void* stream, int dtype);

/*
 * The number of key ranges for fa_fwd_split on the current device: with U =
 * B * H * ceil(N / tile_q) the plain launch's (head, query tile) units and C
 * the device's compute units, floor(C / U) without the mask (ranges that
 * bring the units up to one per CU) and floor(2 C / U) under it (a causal
 * launch with fewer than 2 C units waits on its longest rows), clamped to
 * [1, min(16, key tiles)].  1 means that the plain fa_fwd is the faster
 * call.  Writes *splits; FA_ERR_INVALID for a null pointer, a size <= 0 or
 * causal not 0 or 1, FA_ERR_UNSUPPORTED for another dtype or d, FA_ERR_HIP
 * if the device query fails (no HIP launch is made).
 */
int fa_fwd_split_count(int B, int H, int N, int d, int causal, int dtype, int* splits);

/*
 * The (tile_q, tile_k) shape of the per-tile kernel for these parameters:
 * the tile of fp32-output launches and of launches too small for the
 * persistent kernels (fa_fwd_launch_tile gives the tile of any launch).
 * Pure host function, no HIP call.  Returns FA_OK, or FA_ERR_UNSUPPORTED /
 * FA_ERR_INVALID with the outputs untouched.
 */
int fa_fwd_tile_shape(int dtype, int d, int causal, int* tile_q, int* tile_k);

/*
 * The (tile_q, tile_k) tile that fa_fwd_ex(args) would work in on the
 * current device -- the unit of its tile counters, so that the caller can
 * compute the expected counts for exactly that tiling (block counting of
 * §2.2 of "FlashAttention分块计算优化Transformer显存效率" at B_q = tile_q,
 * B_k = tile_k).  The choice depends on B * H, N, the mask, the output type
 * and the device's compute-unit count: 16-bit launches at d = 128 that fill
 * the device run persistent kernels (256 x 64 tiles under either mask), the
 * others the per-tile kernels (fa_fwd_tile_shape: 256 x 64 without a mask
 * and 128 x 64 causal at d = 128, 128 x 64 at d = 64, 64 x 64 in fp32).  A launch with counters runs the instrumented
 * instance of the kernel the same launch without counters runs.
 * Nothing is launched; args->counters is not read.  The arguments are
 * checked as by fa_fwd_ex (same error codes); then the device is queried
 * (cached): FA_ERR_UNSUPPORTED if it is not gfx950, FA_ERR_HIP if the query
 * fails.  FA_ERR_INVALID for a NULL tile_q or tile_k.
 */
int fa_fwd_launch_tile(const fa_fwd_args* args, int* tile_q, int* tile_k);

/* Static description of a status code; never NULL. */
const char* fa_strerror(int status);

/* Static description of the build: offload architecture, compile flags and
 * the kernel instances built.  Never NULL. */
const char* fa_build_info(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_FWD_H */
