/*
 * fa_probe.h -- clock probe for measuring the forward's launches.
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

#ifdef __cplusplus
}
#endif

#endif /* FA_PROBE_H */
