/*
 * fa_bwd.h -- C ABI of the attention backward pass with recomputation.
 *
 * "Flash Attention 原理" names recomputation as the method's second pillar:
 * the forward pass keeps each row's softmax statistics instead of the N x N
 * probability matrix, and the backward pass rebuilds the probabilities tile
 * by tile from them.  Here the kept statistic is the forward's per-row
 * log-sum-exp (fa_fwd.h), so that for every head
 *
 *   P      = exp(scale * Q K^T - LSE)            (rebuilt per tile, never stored;
 *                                                 0 where key > query when causal)
 *   D[i]   = sum_c dO[i,c] O[i,c]                (= sum_j P[i,j] dP[i,j])
 *   dV     = P^T dO
 *   dP     = dO V^T
 *   dS     = P * (dP - D)                        (row-wise softmax Jacobian)
 *   dQ     = scale * dS K
 *   dK     = scale * dS^T Q
 *
 * the gradients of the forward O = softmax(scale Q K^T [causal]) V of
 * "FlashAttention分块计算优化Transformer显存效率" §1.1 and §2.2 at the output
 * gradient dO.
 *
 * Entry points (one per element type, plus a generic form with a trailing
 * dtype as in fa_fwd.h).  bf16 and fp16 run the 16-bit matrix-core products
 * with P and dS rounded to the input type and fp32 accumulation; fp32 runs
 * fp32 matrix-core products throughout and writes fp32 gradients.
 *
 *   q, k, v, o, dout : device, const, dense row-major [B, H, N, d] of the
 *                      element type; o and lse are the forward's outputs for
 *                      the same q, k, v, scale and causal.
 *   lse              : device, const, [B, H, N] fp32 (natural log).
 *   dq, dk, dv       : device, written, [B, H, N] x d of the element type.
 *   delta            : device, written, [B, H, N] fp32 work array (D above);
 *                      the caller allocates it, the library allocates nothing.
 *   B, H, N, d       : sizes; d = 64 or 128.
 *   scale, causal    : as in the forward call.
 *   stream           : hipStream_t as an opaque pointer; work is enqueued on
 *                      it (two kernels: dQ and D first, then dK and dV) and
 *                      the call returns without synchronising.
 *
 * Ownership: the caller owns every buffer.  The outputs and delta must not
 * overlap any input or each other; the inputs may alias one another.
 *
 * Errors (fa_status of fa_fwd.h); every check runs before any HIP call:
 * FA_ERR_INVALID for a null pointer, B, H, N or d <= 0, causal not 0 or 1, a
 * non-finite scale, or an output overlapping an input or another output;
 * FA_ERR_UNSUPPORTED for another element type, d other
 * than 64 or 128, N * d * 4 of 2^31 or more (as for fa_fwd), a grid beyond 2^31
 * workgroups, or a current device that is not gfx950; FA_ERR_HIP if the
 * device query or a launch fails.  Faults inside a kernel surface
 * at the caller's next synchronisation.
 */
#ifndef FA_BWD_H
#define FA_BWD_H

#ifdef __cplusplus
extern "C" {
#endif

int fa_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                void* dq, void* dk, void* dv, float* delta, int B, int H, int N, int d, float scale, int causal,
                void* stream);
int fa_bwd_f16(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
               void* dq, void* dk, void* dv, float* delta, int B, int H, int N, int d, float scale, int causal,
               void* stream);
int fa_bwd_f32(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
               void* dq, void* dk, void* dv, float* delta, int B, int H, int N, int d, float scale, int causal,
               void* stream);
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout, void* dq,
           void* dk, void* dv, float* delta, int B, int H, int N, int d, float scale, int causal, void* stream,
           int dtype);

/*
 * fa_bwd with O in fp32: o is a dense row-major [B, H, N, d] fp32 array (the
 * forward's fp32 output, fa_fwd_ex with out_dtype = 1) whatever dtype says;
 * every other argument, the layout of the rest and the errors are those of
 * fa_bwd.  O enters the backward only through D[i] = sum_c dO[i,c] O[i,c]
 * (the identity D[i] = sum_j P[i,j] dP[i,j] above, which holds for the exact
 * O); from a 16-bit O, D carries that O's rounding (relative 2^-9 in bf16 per
 * element), and dS = P * (dP - D) magnifies it wherever dP - D is small.
 * From the fp32 O, D is as accurate as the forward's fp32 accumulators.
 * With o holding exactly the values of a 16-bit O the result equals
 * fa_bwd's bit for bit.  dtype FA_DTYPE_F32 is fa_bwd itself.
 */
int fa_bwd_o32(const void* q, const void* k, const void* v, const float* o, const float* lse, const void* dout,
               void* dq, void* dk, void* dv, float* delta, int B, int H, int N, int d, float scale, int causal,
               void* stream, int dtype);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): fa_bwd
 * without the delta argument.  The D work array lives in a fixed scratch
 * array inside the library, FA_BWD_NOALLOC_MAX_ROWS fp32 values (16 MiB),
 * one copy per device, held until the process ends; its address is resolved
 * on the first call made with that device current.  The call allocates
 * nothing and runs the same kernels as fa_bwd, so it returns the same bits.
 *   B * H * N above FA_BWD_NOALLOC_MAX_ROWS -> FA_ERR_SCRATCH, before any HIP
 *   call; every other argument and error as for fa_bwd.
 * All calls on one device share that device's scratch array: calls that
 * overlap in time on one device (different streams, or host threads without
 * ordering) race on it and must be serialised by the caller.  Nothing in the
 * array needs to start at zero; each call writes D before reading it.
 */
#define FA_BWD_NOALLOC_MAX_ROWS (1 << 22)
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                   void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, void* stream,
                   int dtype);

#ifdef __cplusplus
}
#endif

#endif
