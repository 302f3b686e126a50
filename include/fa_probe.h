/*
 * fa_probe.h -- probes for measuring the forward's launches: the shader
 * clock, and the issue rates of the key loop's instruction mixes.
 *
 * The forward's throughput on MI355X depends on the shader clock the chip
 * holds under load (it is power-limited), and that clock changes from launch
 * to launch while the power manager settles.  A probe enqueued right after
 * (or before) a stretch of work on a stream measures the shader clock at that
 * moment: FA_PROBE_WAVES single-wave workgroups each count their CU's shader
 * cycles (s_memtime) over `ticks` ticks of the constant-rate real-time
 * counter (s_memrealtime, whose rate is hipDeviceAttributeWallClockRate, in
 * kHz), so that
 *
 *   shader clock = cycles / ticks * tick_rate
 *
 * per wave.  The power manager reacts over milliseconds, so a probe of tens
 * of microseconds reads the clock the preceding work ran at.
 *
 *   out     device pointer to 2 * FA_PROBE_WAVES unsigned 64-bit integers,
 *           written: out[2w] = shader cycles counted by wave w, out[2w + 1] =
 *           real-time ticks over which they were counted (>= ticks).
 *   ticks   real-time ticks to count over, 1 .. FA_PROBE_MAX_TICKS (at the
 *           MI355X's 100 MHz, 2000 ticks = 20 us); every wave waits until
 *           the real-time counter has advanced that far, so the kernel ends.
 *   stream  hipStream_t as an opaque pointer (NULL: default stream); the call
 *           enqueues the probe kernel and returns without synchronising.
 *
 * Returns FA_ERR_INVALID for a NULL out or ticks out of range (before any
 * HIP call), FA_ERR_UNSUPPORTED if the current device is not gfx950,
 * FA_ERR_HIP if the launch fails, FA_OK otherwise (fa_status of fa_fwd.h).
 * The caller owns out.
 */
#ifndef FA_PROBE_H
#define FA_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

#define FA_PROBE_WAVES 64
#define FA_PROBE_MAX_TICKS 1000000
int fa_clock_probe(unsigned long long* out, unsigned ticks, void* stream);

/*
 * Issue-rate probe: the instruction mixes of the forward's key loop, without
 * its memory traffic, LDS reads or barriers, on every SIMD of the device --
 * two four-wave workgroups per CU, so two waves per SIMD as in the kernels
 * -- to measure what the VALU and the matrix cores sustain together.  Each
 * wave runs `iters` iterations of one mix on register data; per iteration it
 * issues (the modes):
 *   FA_PROBE_EXP       16 v_exp_f32
 *   FA_PROBE_FMA       16 v_fma_f32
 *   FA_PROBE_ADD       16 v_add_f32
 *   FA_PROBE_PACK      8 v_cvt_pk_bf16_f32 (+ 8 xor that keep them live)
 *   FA_PROBE_SOFTMAX   4 softmax pairs: 2 fma, 2 exp, 1 pack (+ xor), 2 add
 *                      each -- the work the kernels spend on two scores
 *   FA_PROBE_MFMA      4 v_mfma_f32_32x32x16_bf16 on 4 accumulators
 *   FA_PROBE_MIX64     4 MFMA + 4 softmax pairs (the ratio at d = 64)
 *   FA_PROBE_MIX128    4 MFMA + 2 softmax pairs (the ratio at d = 128)
 *
 *   out      device pointer to out_len unsigned 64-bit integers; wave w of
 *            the grid writes out[3w] = shader cycle counter ticks between
 *            its start and end, out[3w + 1] / out[3w + 2] = the real-time
 *            counter at its start / end.  The grid has 8 * CUs waves; out_len
 *            must be at least 3 * 8 * CUs.
 *   iters    1 .. FA_PROBE_MAX_ITERS
 *   stream   hipStream_t as an opaque pointer; returns without synchronising.
 * The chip-level time per instruction per SIMD is
 *   (latest end - earliest start) / tick rate * SIMDs / (waves * iters * n)
 * with n the count above.  Errors: FA_ERR_INVALID for a NULL out, a mode or
 * iters out of range, or out_len too small (before any HIP call, except the
 * device query that gives the CU count); FA_ERR_UNSUPPORTED off gfx950;
 * FA_ERR_HIP if the launch fails.
 */
enum {
    FA_PROBE_EXP = 0, FA_PROBE_FMA = 1, FA_PROBE_ADD = 2, FA_PROBE_PACK = 3, FA_PROBE_SOFTMAX = 4,
    FA_PROBE_MFMA = 5, FA_PROBE_MIX64 = 6, FA_PROBE_MIX128 = 7, FA_PROBE_MODES = 8
};
#define FA_PROBE_MAX_ITERS 1000000
int fa_issue_probe(int mode, int iters, unsigned long long* out, long long out_len, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_PROBE_H */
