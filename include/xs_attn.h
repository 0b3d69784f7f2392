/*
 * xs_attn.h -- C ABI of the fused attention + destination-ordered epilogue
 * library for AMD Instinct MI355X (gfx950).
 *
 * The operation (X-Stage paper, "X-Stage: An Overlooked Pipeline Stage for
 * Communication-Computation Overlap in DiT Inference": catalyzex.com abstract;
 * gist.science explainer, section "Zentrale Beitraege", item
 * "FlashAttention-A2A (Piggybacking)"): one GPU's share of Ulysses
 * sequence-parallel attention in a Diffusion Transformer -- the full sequence
 * S over H_local heads -- computed as a non-causal FlashAttention forward pass
 * whose output-tile owner writes each finished O tile straight into the buffer
 * the post-attention All-to-All would deliver, with no dedicated communication
 * wavefront.  Here that buffer lives in the calling GPU's own HBM.
 *
 *   O[b,s,h,:] = softmax_j(scale * q[b,s,h,:] . k[b,j,h,:]) @ v[b,:,h,:]
 *   out_packed[p][b][s'][h][d] = O[b][p*T + s'][h][d],   T = S / P
 *   (flat offset (((p*B + b)*T + s')*H_local + h)*D + d)
 *
 * Conventions shared by every entry point:
 *  - q, k, v are device pointers to contiguous [B][S][H_local][D] tensors.
 *  - out_packed is a device pointer to a contiguous [P][B][S/P][H_local][D]
 *    bf16 tensor; it must not overlap q, k or v.
 *  - All device pointers must be 16-byte aligned.
 *  - The caller owns every buffer.  The library allocates nothing, keeps no
 *    pointer after returning, holds no global state and is re-entrant.
 *  - `stream` is a hipStream_t passed as void*; NULL selects the default
 *    stream.  Calls are asynchronous: they return once the kernel is enqueued
 *    and do not synchronise; a fault inside the kernel surfaces at the
 *    caller's next synchronisation on that stream.
 *  - Arguments are validated before any HIP call, so validation errors are
 *    reported (and testable) without a GPU.  No entry point prints, throws or
 *    aborts.
 */
#ifndef XS_ATTN_H
#define XS_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
#define XS_OK 0
#define XS_ERR_NULL (-1)        /* a required pointer is NULL */
#define XS_ERR_SHAPE (-2)       /* B, S, H_local, D or P < 1, or S % P != 0 */
#define XS_ERR_UNSUPPORTED (-3) /* D not in {64, 128}, scale or a descale not finite,
                                   S*H_local*D*elem_bytes >= 4 GiB (one batch's rows), an
                                   unknown input layout, or chunked inputs with B > 1, P > 1
                                   and S/P not a multiple of 64 */
#define XS_ERR_ALIGN (-4)       /* a pointer is not 16-byte aligned */
#define XS_ERR_LAUNCH (-5)      /* the HIP launch reported an error */
#define XS_ERR_OVERLAP (-6)     /* out_packed, lse or the workspace overlaps another buffer */
#define XS_ERR_WORKSPACE (-7)   /* workspace smaller than xs_attn_workspace_size() */
#define XS_ERR_SCRATCH (-8)     /* xs_attn_fwd_noalloc: partials exceed its static scratch */
/* (XS_ERR_UNSUPPORTED also when B*H_local*ceil(S/128) exceeds 2^31 - 1 half-height query
   tiles.) */

/* Attention forward over bf16 inputs with the destination-ordered epilogue.
 *   q, k, v     bf16 [B][S][H_local][D], device memory (read only)
 *   out_packed  bf16 [P][B][S/P][H_local][D], device memory (written fully)
 *   scale       fp32 softmax scale applied to the fp32 dot products
 *               (1/sqrt(D) for standard attention); any finite value.
 * Accumulation is fp32; the probabilities enter the second contraction as
 * bf16; the output is rounded to bf16 (round to nearest even). */
int xs_attn_fwd(const void *q, const void *k, const void *v, void *out_packed, int B, int S,
                int H_local, int D, int P, float scale, void *stream);

/* The same operation over OCP fp8 e4m3 (e4m3fn) inputs with per-tensor fp32
 * descales: the value of element x is x8 * x_descale.  The e4m3 matrix cores
 * accumulate into fp32, though a dot product's terms are not summed to full
 * fp32 precision (measured: up to about 2^-12.8 of scale * sum_d |q_d k_d| when
 * one product dominates); the probabilities enter the second contraction as
 * e4m3 codes read off their exponents (for p = 2^y, the code of 2^e (1 + f) with
 * e + f = y, rounded to e4m3's three mantissa bits: within 12.8 % of a common
 * multiple of p, no exponential is evaluated), and O is normalised by the sum of
 * those quantised probabilities (a constant V comes back exactly).  The output
 * is bf16 [P][B][S/P][H_local][D] as above.  Descales must be finite. */
int xs_attn_fwd_fp8(const void *q8, const void *k8, const void *v8, float q_descale,
                    float k_descale, float v_descale, void *out_packed, int B, int S, int H_local,
                    int D, int P, float scale, void *stream);

/* Scheduled variants.  The work of a call is a sequence of units (one 256-row
 * query tile x two 64-key blocks).  The library chooses, per shape and device, a
 * number of workgroups that share the units equally: one per tile (nothing to
 * merge), k equal key-range pieces per tile, or one persistent workgroup per
 * compute unit walking an equal contiguous share -- so tile outputs finish at
 * staggered times rather than in lockstep rounds, and a workgroup requests its
 * next tile's first K/V blocks and queries before it stores the current one
 * (X-Stage paper, gist.science explainer, "FlashAttention-A2A (Piggybacking)":
 * the tile owner stores its output and immediately resumes the next tile's
 * loop).  A tile whose key range is shared by several workgroups is cut: each
 * piece writes unnormalised fp32 partials (O and, per row, the running max and
 * row sum) into `workspace`, and a second kernel on the same stream merges them
 * with the online-softmax rule into out_packed -- the merge of partial
 * attention by online softmax of "Move the Query, Not the Cache" (gist.science
 * explainer, Methodik: the Route primitive), applied inside one GPU.
 *   workspace        device memory, 16-byte aligned, at least
 *                    xs_attn_workspace_size(B, S, H_local, D) bytes; owned by the
 *                    caller, not retained after the call; its contents are
 *                    scratch (overwritten, never read before written).  Calls
 *                    that overlap in time must not share a workspace.  When the
 *                    schedule cuts tiles, the workspace_size bytes it uses may
 *                    not overlap q, k, v, out_packed or lse (XS_ERR_OVERLAP).
 *   workspace NULL   no tile is cut (identical to xs_attn_fwd).
 * Results differ from the uncut schedule only by rounding (pieces are merged in
 * key order, so they are deterministic); they do not depend on P.
 * Returns XS_ERR_WORKSPACE if workspace is non-NULL but too small. */
int xs_attn_fwd_ws(const void *q, const void *k, const void *v, void *out_packed, int B, int S,
                   int H_local, int D, int P, float scale, void *workspace,
                   size_t workspace_bytes, void *stream);
int xs_attn_fwd_fp8_ws(const void *q8, const void *k8, const void *v8, float q_descale,
                       float k_descale, float v_descale, void *out_packed, int B, int S,
                       int H_local, int D, int P, float scale, void *workspace,
                       size_t workspace_bytes, void *stream);

/* For callers that cannot allocate (code under HIP-graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): xs_attn_fwd_ws without the
 * workspace arguments.  The split-key partials go to a static device array of
 * the library, XS_NOALLOC_SCRATCH_BYTES bytes (65 MiB) that every GPU the
 * library runs on holds until the process ends; the call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine).  The first call on a
 * device looks up that device's copy of the array (hipGetSymbolAddress) and
 * keeps its address.  65 MiB holds the partials of every shape on a device of
 * up to 256 compute units (at most one workgroup per compute unit writes two
 * 256-row slots of fp32 O, max and sum); a larger need returns XS_ERR_SCRATCH
 * before any launch.  The partials are always written before they are read,
 * so nothing has to start at zero.  Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (on different streams, or from
 * different threads without ordering) race and give wrong results; calls
 * ordered on one stream do not.  Arguments, results and status codes are
 * those of xs_attn_fwd_ws (bit-identical output for the same inputs). */
#define XS_NOALLOC_SCRATCH_BYTES 68157440
int xs_attn_fwd_noalloc(const void *q, const void *k, const void *v, void *out_packed, int B,
                        int S, int H_local, int D, int P, float scale, void *stream);

/* Input layouts of q, k, v for the _ex entry points. */
#define XS_LAYOUT_BSHD 0    /* [B][S][H_local][D] */
#define XS_LAYOUT_CHUNKED 1 /* [P][B][S/P][H_local][D]: chunk p holds rows p*T .. p*T+T-1
                               (T = S/P) of every batch -- the layout the Ulysses
                               pre-attention All-to-All delivers, the same chunk layout as
                               out_packed.  Byte-identical to BSHD when B = 1 or P = 1. */
/* Flag OR-ed into in_layout: run the whole call in one attention launch, as a call
 * whose out_packed lies behind a link does (no half-height tiles in a second launch,
 * xs_attn_schedule_ex); the rows are the same bit for bit.  For comparing an output
 * in device memory with one behind a link under the same schedule. */
#define XS_ONE_LAUNCH 0x100

/* The split-key entry points with two additions (both optional):
 *   in_layout  XS_LAYOUT_BSHD or XS_LAYOUT_CHUNKED: q, k, v may be consumed directly
 *              in the chunk layout the pre-attention All-to-All of Ulysses sequence
 *              parallelism delivers (X-Stage paper, catalyzex.com abstract: Ulysses
 *              sequence-parallel attention between two All-to-Alls; gist.science
 *              explainer, "FlashAttention-A2A (Piggybacking)"), so no relayout pass
 *              runs before attention.  With B > 1 and P > 1, S/P must be a multiple
 *              of 64 (XS_ERR_UNSUPPORTED otherwise).
 *   lse        NULL, or device memory for [B][H_local][S] fp32 (4-byte aligned, not
 *              overlapping q, k, v or out_packed, else XS_ERR_ALIGN / XS_ERR_OVERLAP):
 *              receives the natural-log log-sum-exp of every query row,
 *              lse = log(sum_j exp(scale * q.k_j)) (for fp8, scale*dq*dk * q8.k8_j),
 *              the quantity an online-softmax merge of partial attention needs
 *              ("Move the Query, Not the Cache", gist.science explainer, Methodik:
 *              the Route primitive).  It is the running max plus log of the row sum
 *              of the kernel's own softmax, taken over the fp32 probabilities
 *              before their rounding to bf16 / e4m3.  For fp8 with lse, P is
 *              2^(s c - m) rounded to the nearest e4m3 and O is normalised by
 *              that fp32 sum too (it differs from the call without lse within
 *              the two encodings of P); for bf16, O is the same with or without
 *              lse.
 * Every other argument, the workspace rules and the error behaviour are those of
 * xs_attn_fwd_ws / xs_attn_fwd_fp8_ws, which equal these calls with in_layout =
 * XS_LAYOUT_BSHD and lse = NULL. */
int xs_attn_fwd_ex(const void *q, const void *k, const void *v, int in_layout, void *out_packed,
                   float *lse, int B, int S, int H_local, int D, int P, float scale,
                   void *workspace, size_t workspace_bytes, void *stream);
int xs_attn_fwd_fp8_ex(const void *q8, const void *k8, const void *v8, int in_layout,
                       float q_descale, float k_descale, float v_descale, void *out_packed,
                       float *lse, int B, int S, int H_local, int D, int P, float scale,
                       void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace the scheduled variants need on the current device for this
 * shape (0: no tile is cut).  Depends on the device's compute-unit count;
 * returns 0 for invalid sizes.  No allocation, no kernel launch. */
size_t xs_attn_workspace_size(int B, int S, int H_local, int D);

/* The most pieces the scheduled variants cut any query tile into for this shape
 * on the current device (1 = no tile is cut); 0 for invalid sizes. */
int xs_attn_split_count(int B, int S, int H_local, int D);

/* The schedule the library runs for a call of this shape on the current
 * device, with (with_workspace != 0) or without a workspace:
 * xs_attn_schedule_ex(B, S, H_local, D, with_workspace, 0, groups, whole_rounds,
 * pieces, NULL). */
int xs_attn_schedule(int B, int S, int H_local, int D, int with_workspace, int *groups,
                     int *whole_rounds, int *pieces);

/* The schedule the library runs for this shape on the current device, for a
 * bf16 (fp8 = 0) or fp8 (fp8 != 0) call -- the two are scheduled alike -- with
 * (with_workspace != 0) or without a workspace.  Work is split into query tiles of 256 rows (8 wavefronts of 32
 * rows each) and, inside a tile, pairs of 64-key blocks:
 *   groups        workgroups of the first launch (0 when it has none);
 *   whole_rounds  rounds of whole tiles each of them takes first;
 *   pieces        the most pieces any remaining tile is cut into by their
 *                 shares of its key blocks (1 = none is cut; cut tiles are
 *                 merged by a second kernel);
 *   half_tiles    calls whose schedule cuts no tile and leaves at most half
 *                 a round of tiles after the whole rounds: those tiles run as
 *                 128-row half tiles (4 wavefronts) in a second launch, one
 *                 workgroup each, so that the last round fills the chip
 *                 (0 = none).  Only when out_packed is
 *                 device memory of the current device: behind a link (host or
 *                 peer memory) the first launch would have to drain its whole
 *                 last round before the second starts, so such calls keep a
 *                 last round of full tiles in the same launch (the schedule
 *                 with half_tiles = 0 and groups covering every tile).
 * Any output pointer may be NULL.  Returns XS_OK or XS_ERR_SHAPE (sizes < 1, D
 * not 64 or 128).  No launch. */
int xs_attn_schedule_ex(int B, int S, int H_local, int D, int with_workspace, int fp8,
                        int *groups, int *whole_rounds, int *pieces, int *half_tiles);

/* Static, never-NULL description of a status code. */
const char *xs_attn_strerror(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int xs_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* XS_ATTN_H */
