/*
 * fa_standard.h -- C ABI of the standard (materialising) attention forward
 * built beside fa_fwd as a measured baseline.
 *
 * "FlashAttention分块计算优化Transformer显存效率" §1.1 describes the standard
 * computation that FlashAttention replaces: the N x N score matrix S and the
 * probability matrix P are written to HBM and read back, and §2.1 counts its
 * memory traffic (per head at N = 4096, d = 128, 16-bit: reads Q, K, V, S and
 * P, 67 MiB; writes S, P and O, 65 MiB).  This entry point computes exactly
 * that way, with three plain kernels on the caller's stream:
 *
 *   scores   S = scale * Q K^T                  (N x N, stored in the input type)
 *   softmax  P = row-softmax(S), with the causal mask j > i -> 0,
 *            LSE[i] = ln sum_j exp(S[i,j])      (P stored in the input type)
 *   output   O = P V                            (stored in the input type)
 *
 * so that the traffic of S and P can be measured against the tiled forward of
 * fa_fwd.h, which never stores them.  Same result as fa_fwd up to rounding (S
 * and P are rounded to the input type here).
 *
 * Layout.  q, k, v, o: dense row-major [B, H, N, d]; lse: [B, H, N] fp32;
 * s and p: dense row-major [B, H, N, N] work arrays of the input element
 * type, written by the call (the caller allocates them: 2 * B * H * N * N
 * elements in all; the library allocates nothing).
 *
 * Types and sizes.  dtype FA_DTYPE_BF16 or FA_DTYPE_F16 (fa_fwd.h); d = 64 or
 * 128; B, H, N > 0; N * d * 4 below 2^31 (as for fa_fwd).
 *
 * Errors (fa_status of fa_fwd.h).  Every check runs before any HIP call:
 * FA_ERR_INVALID for null pointers, s or p not 16-byte aligned, B, H, N or
 * d <= 0, causal not 0 or 1, a non-finite scale; FA_ERR_UNSUPPORTED for another element type or d,
 * sizes beyond the above, or a current device that is not gfx950.  FA_ERR_HIP if the device query
 * or a launch fails.  The call returns
 * without synchronising.
 */
#ifndef FA_STANDARD_H
#define FA_STANDARD_H

#ifdef __cplusplus
extern "C" {
#endif

int fa_standard_fwd(const void* q, const void* k, const void* v, void* o, float* lse, void* s, void* p,
                    int B, int H, int N, int d, float scale, int causal, void* stream, int dtype);

#ifdef __cplusplus
}
#endif

#endif
