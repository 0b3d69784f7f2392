/*
 * xs_ceiling.h -- C ABI of the matrix-core ceiling probes of the same library
 * (libxs_attn.so): how fast one gfx950 SIMD issues v_mfma_f32_32x32x16_bf16
 * while it also streams the LDS operand reads and the vector work that the
 * attention kernels put next to each MFMA.
 *
 * The attention forward (FlashAttention over the full sequence of this GPU's
 * Ulysses share: X-Stage paper, gist.science explainer, "Zentrale Beitraege",
 * "FlashAttention-A2A (Piggybacking)") is bound by the matrix cores, but each
 * MFMA of the bf16 kernel needs 1 KiB of operand data from LDS (32 query rows
 * per wave) and about three vector instructions and one exponential of
 * softmax work.  These probes measure the MFMA rate the chip sustains under
 * each stream alone and under both, so the kernel's own MFMA-busy fraction
 * can be read against them.  Modes 0-6 multiply fixed or arbitrary bit
 * patterns (little switching activity, and NaN once an accumulator overflows);
 * modes 7-12 use data distributed like the workloads' inputs, which draws
 * the power that real inputs draw.
 */
#ifndef XS_CEILING_H
#define XS_CEILING_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define XS_CEIL_MFMA 0      /* MFMAs only, four independent accumulators per wave */
#define XS_CEIL_LDS_1K 1    /* + one 1 KiB ds_read_b128 per MFMA, read three MFMAs ahead */
#define XS_CEIL_LDS_HALF 2  /* + one 1 KiB ds_read_b128 per two MFMAs (0.5 KiB per MFMA) */
#define XS_CEIL_TR16_1K 3   /* + two 512-byte ds_read_b64_tr_b16 per MFMA, three MFMAs ahead */
#define XS_CEIL_SOFTMAX 4   /* + the bf16 kernel's softmax work per MFMA: one v_fma_f32, one
                               v_exp_f32, one v_add_f32 and half a v_cvt_pk_bf16_f32, no LDS */
#define XS_CEIL_MIX 5       /* XS_CEIL_SOFTMAX + XS_CEIL_LDS_1K: the mix of 32 query rows per wave */
#define XS_CEIL_MIX_HALF 6  /* XS_CEIL_SOFTMAX + XS_CEIL_LDS_HALF: the mix of 64 query rows per wave */
#define XS_CEIL_MFMA_DATA 7  /* XS_CEIL_MFMA with operands like the bf16 workloads' inputs: A and B
                               rotate through eight register-held fragments of N(0, 1) draws in
                               bf16, so every MFMA switches operand bits as the attention kernel's do */
#define XS_CEIL_MIX_DATA 8   /* XS_CEIL_MIX on such data: the LDS holds those values, the softmax
                               stand-in takes a new argument per MFMA (the A operand's first word
                               read as fp32) and its probabilities, 2^(1.44 x - 5) as the video
                               share's scores relative to their running max, are the B operand */
#define XS_CEIL_MFMA16_DATA 9 /* XS_CEIL_MFMA_DATA with each 32x32x16 MFMA replaced by two
                               v_mfma_f32_16x16x32_bf16 (the same multiply-adds; a quarter of
                               the accumulator registers read and written per instruction) */
#define XS_CEIL_MIX16_DATA 10 /* XS_CEIL_MIX_DATA with each 32x32x16 MFMA replaced by two
                               v_mfma_f32_16x16x32_bf16 that share the LDS fragment as A operand
                               (two 16-query tiles; the second's B operand is the next MFMA's
                               LDS fragment, random data already in registers) */
#define XS_CEIL_FP8_DATA 11     /* v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3, 64 clocks, four times
                                   the multiply-adds of one bf16 MFMA) alone on operands like the fp8
                                   workload's (N(0, 1) draws quantised to e4m3 with amax 5 -> 448),
                                   rotating through eight register-held fragments */
#define XS_CEIL_FP8_MIX_DATA 12 /* the fp8 kernel's per-MFMA mix on such data: 2 KiB of LDS operand
                                   (two ds_read_b128) as A, and as B e4m3 codes made per MFMA by
                                   four FMAs, two v_cvt_pknorm_u16_f32, one v_perm_b32 and two
                                   three-input maxima from an earlier accumulator (codes 54 +- 12,
                                   as the fp8 share's probabilities) */
#define XS_CEIL_MODES 13

#define XS_CEIL_SINK_BYTES (1024u * 512u * 4u) /* smallest sink accepted */

#define XS_CEIL_ERR_NULL (-1)   /* sink is NULL */
#define XS_CEIL_ERR_ARG (-2)    /* mode, waves_per_simd or iters out of range */
#define XS_CEIL_ERR_SIZE (-3)   /* sink_bytes below XS_CEIL_SINK_BYTES */
#define XS_CEIL_ERR_ALIGN (-4)  /* sink not 4-byte aligned */
#define XS_CEIL_ERR_LAUNCH (-5) /* the HIP launch reported an error */

/* Launches one probe kernel: 1024 workgroups of 256*waves_per_simd threads (one
 * workgroup per compute unit at a time, so each SIMD runs waves_per_simd waves),
 * every wave issuing 16*iters MFMAs together with the mode's stream.  LDS
 * addresses stay inside a 64 KiB array that each workgroup fills first; every
 * other operand lives in registers.  Each thread stores one float into sink
 * (thread t of workgroup g at index g*512 + t) so that none of the work is dead;
 * the values carry no meaning.
 *   mode            XS_CEIL_* (0 .. XS_CEIL_MODES-1)
 *   waves_per_simd  1 or 2
 *   iters           1 .. 2^20
 *   sink            device memory, at least XS_CEIL_SINK_BYTES bytes, 4-byte aligned
 *   stream          hipStream_t as void*, NULL = default stream; asynchronous:
 *                   time it with events on the same stream.
 * A run issues 1024/256 * waves_per_simd * 16 * iters MFMAs per SIMD (256
 * compute units, 4 SIMDs each), 32 shader clocks each at full rate.
 * Returns 0 or an XS_CEIL_ERR_* code (validated before any HIP call). */
int xs_mfma_ceiling(int mode, int waves_per_simd, int iters, float *sink, size_t sink_bytes, void *stream);

/* Shader clock under a timed run.  The chip sets its clock by the power a kernel
 * draws, so the clock a run actually held decides how its rate compares with the
 * published peak (which assumes 2.4 GHz).  Launches one small kernel on `stream`:
 * XS_CLOCK_GROUPS workgroups of one wave (several per compute unit); wave g
 * stores, at out[4g .. 4g+3], its s_memtime (shader clock cycles), its
 * s_memrealtime (a constant-rate counter of *wall_khz kHz), its XCC id (hardware
 * register XCC_ID) and its HW_ID register (compute unit, shader array and shader
 * engine in bits 8-15).  The shader-clock counters of different engines are not
 * synchronised, so a sample taken before and one taken after the timed launches on
 * the same stream are paired per compute unit (XCC and HW_ID bits 8-15): there
 * (memtime difference) / (realtime difference) * wall_khz kHz = the mean shader
 * clock over the interval.
 *   out       device memory, at least XS_CLOCK_BYTES bytes, 8-byte aligned
 *   wall_khz  host int: the constant counter's rate (hipDeviceAttributeWallClockRate)
 *   stream    hipStream_t as void*, NULL = default stream; asynchronous
 * Returns 0, XS_CEIL_ERR_NULL, XS_CEIL_ERR_SIZE, XS_CEIL_ERR_ALIGN or
 * XS_CEIL_ERR_LAUNCH (arguments validated before any HIP call). */
#define XS_CLOCK_GROUPS 1024
#define XS_CLOCK_BYTES (XS_CLOCK_GROUPS * 4u * 8u)
int xs_clock_sample(unsigned long long *out, size_t out_bytes, int *wall_khz, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* XS_CEILING_H */
