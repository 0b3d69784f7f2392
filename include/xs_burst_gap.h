/*
 * xs_burst_gap.h -- C ABI of the Burst-Gap microbenchmark of the same library
 * (libxs_attn.so), for characterising how device-issued store bursts drain on
 * one GPU.
 *
 * What it measures (X-Stage paper, gist.science explainer, "Methodik: Die
 * X-Stage-Abstraktion und das Burst-Gap-Modell" and "Zentrale Beitraege",
 * item "Charakterisierung und Vorhersage"): K producers each issue a burst of
 * stores, then compute for a gap G without memory traffic, and repeat.  The
 * sender-visible issue time of a burst of aggregate volume V is modelled as
 *   T_iss(G; K, V) = max(T0_iss(K, V), V/R - G)
 * with T0_iss the backpressure-free issue time, R the effective drain rate and
 * Q the outstanding capacity.  The pages measure remote stores over a GPU
 * interconnect; on one GPU the destination is any device-accessible memory --
 * fine-grained host memory stands in for the remote link.
 */
#ifndef XS_BURST_GAP_H
#define XS_BURST_GAP_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define XS_BG_ERR_NULL (-1)   /* dst or times is NULL */
#define XS_BG_ERR_ARG (-2)    /* a size out of range (see below) */
#define XS_BG_ERR_ALIGN (-4)  /* dst not 16-byte or times not 8-byte aligned */
#define XS_BG_ERR_LAUNCH (-5) /* the HIP launch reported an error */

/* Runs `producers` workgroups of 256 threads.  dst is used as a ring of
 * ring = min(nburst, floor(dst_bytes / (producers*bytes))) regions of
 * producers*bytes bytes; in burst b, producer p stores all `bytes` bytes of
 * [(r*producers + p)*bytes, (r*producers + p + 1)*bytes), r = b % ring (16
 * bytes per lane per step, fully coalesced; the 16 bytes lane t writes are the
 * uint32 words {p, t, b, 0x5eed}), then spins `gap_cycles` shader clocks
 * without memory traffic.  A ring of nburst regions makes every burst write
 * fresh addresses, as output tiles do.
 *   dst         device-accessible memory of at least producers*bytes bytes,
 *               16-byte aligned; bytes past the ring are not touched.
 *   producers   1 .. 4096
 *   bytes       per producer and burst: a multiple of 4096, at most 1 GiB
 *   nburst      1 .. 4096
 *   gap_cycles  0 .. 2^32 shader clocks, and nburst*gap_cycles <= 2^34 (a
 *               run of seconds at most)
 *   times       device memory, 8-byte aligned, producers*4*(nburst+3) uint64:
 *               for producer p and wave w (4 per producer) the record at
 *               (p*4 + w)*(nburst+3) holds, in shader clocks (s_memtime), the
 *               issue time of each burst (first store to issue of the last
 *               store, no wait for completion), then the time its stores took
 *               to complete after the last gap, then the clocks of the whole
 *               run, then the same run in 100 MHz ticks (s_memrealtime) --
 *               the last two give the clock rate for converting to seconds.
 *   stream      hipStream_t as void*, NULL = default stream; asynchronous.
 * Returns 0 or an XS_BG_ERR_* code (validated before any HIP call). */
int xs_burst_gap(void *dst, size_t dst_bytes, int producers, size_t bytes, int nburst,
                 long long gap_cycles, unsigned long long *times, void *stream);

/* The same measurement with the store pattern of the attention epilogue, whose
 * bursts are output tiles: a producer is a workgroup of 512 threads (8 waves)
 * owning one tile of 256 rows of row_bytes bytes each, row_pitch bytes apart (the
 * rows of one head in the destination-ordered buffer are H_local*D*2 bytes
 * apart).  Wave w writes rows 32w .. 32w+31 with row_bytes/16 store instructions
 * of 8 bytes per lane: in instruction c, lane l writes bytes 16c + 8(l/32) .. +7
 * of row 32w + l%32 -- 16 bytes into each of 32 rows per instruction, the order
 * in which the attention kernels store a finished tile.  The bytes lane l writes
 * are the uint32 words {producer, burst}.  A burst of producer p in ring region
 * r = b % ring covers [(r*producers + p)*256*row_pitch, +256*row_pitch) of dst,
 * ring = min(nburst, floor(dst_bytes / (producers*256*row_pitch))); bytes
 * between rows are not touched.
 *   producers   1 .. 4096;  nburst 1 .. 4096
 *   row_bytes   16 .. 4096, a multiple of 16 (a tile's row: D * 2 bytes)
 *   row_pitch   row_bytes .. 2^20, a multiple of 16
 *   gap_cycles  as for xs_burst_gap
 *   coupled     0: the recorded time of a burst is its issue time (first store to
 *               issue of the last, no wait); nonzero: each wave waits for its
 *               stores to complete (s_waitcnt vmcnt(0)) before its gap, and the
 *               recorded time runs to that completion -- what a wave pays when it
 *               next waits on its vector-memory counter, as the attention kernels
 *               do before the next tile's first barrier (the wait for that tile's
 *               K/V loads also covers the stores issued before it).
 *   gap_src     NULL: the gap is gap_cycles of computation-free spinning.
 *               Otherwise the gap is what a tile's key loop does to memory: each
 *               wave issues gap_loads loads of 1 KiB (16 bytes per lane) from
 *               gap_src, fresh addresses every burst (offsets wrap at
 *               gap_src_bytes, a power of two >= 4096), and waits for them;
 *               gap_loads 1 .. 65536, gap_src 16-byte aligned device memory.
 *   times       device memory, 8-byte aligned, producers*8*(2*nburst+3) uint64:
 *               for producer p and wave w the record at (p*8 + w)*(2*nburst+3)
 *               holds each burst's time (issue, or completion when coupled),
 *               then each gap's length, then the drain of the last burst, the
 *               shader clocks of the whole run and its 100 MHz ticks.
 * Returns 0 or an XS_BG_ERR_* code (validated before any HIP call). */
int xs_burst_gap_tiles(void *dst, size_t dst_bytes, int producers, int row_bytes, int row_pitch,
                       int nburst, long long gap_cycles, int coupled, const void *gap_src,
                       size_t gap_src_bytes, int gap_loads, unsigned long long *times,
                       void *stream);

#ifdef __cplusplus
}
#endif

#endif /* XS_BURST_GAP_H */
