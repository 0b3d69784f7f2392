/*
 * xs_probe.h -- measurement helper of the same library (libxs_attn.so): the
 * shader clock the GPU ran at over a stretch of work on a stream.
 *
 * Not an operation of the method.  The published matrix-core peaks assume the
 * chip's peak engine clock; under a sustained matrix load the clock is lower
 * (power limit), so the fraction of the published peak a kernel reaches mixes
 * kernel quality with the clock the box held.  Two stamps on one stream, one
 * before and one after the work, give the average shader clock over it.
 */
#ifndef XS_PROBE_H
#define XS_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

#define XS_CLOCK_STAMP_WORDS 256 /* uint64 words one stamp writes */

/* Enqueues on `stream` (hipStream_t as void*, NULL = default) one tiny kernel of
 * 64 single-wave workgroups (blocks are dealt round-robin over the XCDs, so
 * every XCD runs several) that writes, for each workgroup g, the words
 * stamp[4g .. 4g+3] = {shader clock counter (s_memtime), constant-rate counter
 * (s_memrealtime), XCC id, 0}.  `stamp` is device memory of at least
 * XS_CLOCK_STAMP_WORDS uint64, 8-byte aligned.  The average shader clock over
 * the work enqueued between two stamps a and b is, per XCD,
 * (a.memtime - b.memtime) / (a.realtime - b.realtime) * wall_khz kHz, with
 * wall_khz the constant counter's rate, written to *wall_khz when it is not NULL
 * (hipDeviceAttributeWallClockRate of the current device).
 * Returns 0, -1 (stamp NULL), -4 (misaligned) or -5 (launch or attribute query
 * failed). */
int xs_clock_stamp(void *stamp, int *wall_khz, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* XS_PROBE_H */
