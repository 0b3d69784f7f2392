// attn_launch.h -- host-side launchers of the attention kernels (internal to
// the library; the public interface is include/xs_attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xs {

struct AttnArgs {
  const void* q;  // [B][S][H][D], bf16 or e4m3
  const void* k;
  const void* v;
  void* out;      // bf16 [P][B][T][H][D]
  int B, S, H, D, P, T;
  float c;        // |scale| * log2(e), times q_descale * k_descale for fp8
  int neg;        // nonzero when scale < 0: queries are negated as they are loaded
  float o_scale;  // factor applied with 1/l in the epilogue (v_descale for fp8)
  // Work schedule (see Sched below): `groups` workgroups; each first takes
  // `dp` whole tiles, then an equal share of the `units` (query tile, pair of
  // 64-key blocks) units of the remaining tiles.  Tiles cut between two
  // workgroups leave unnormalised fp32 partials (O, and m, l per row) in the
  // workspace slots of those workgroups; attn_combine merges them into out.
  int groups;
  int npair;
  int dp;
  long long units;
  float* ws_o;    // [2*groups][BM*D] fp32 in register order (NULL when no tile is cut)
  float* ws_ml;   // [2*groups][BM][2] fp32: running max (log2 units), row sum
  // Input layout.  Row s of batch b of an input tensor starts at row index
  //   b*batch_rows + s + (chunk_rows ? s / chunk_rows : 0) * jump_rows
  // (in units of H*D elements): [B][S][H][D] has batch_rows = S, chunk_rows =
  // 0; the chunk layout [P][B][T][H][D] has batch_rows = T, chunk_rows = T,
  // jump_rows = (B-1)*T.
  int batch_rows;
  int chunk_rows;
  long long jump_rows;
  float* lse;     // NULL or [B][H][S] fp32 log-sum-exp (natural log)
  // Tile height of this launch: 0 = kBlockM rows (8 waves), 1 = kBlockM / 2
  // rows (4 waves, whole tiles only).  Tiles are numbered in the
  // launch's own height, tile = (b*H + h) * ceil(S / height) + m-tile, and the
  // launch's schedule starts at tile `tile0` (0 unless an earlier launch of the
  // same call took the tiles before it).
  int half;
  int tile0;
};

// Tile geometry shared by the bf16 and fp8 kernels and the host-side plan.
#ifndef XS_BM
#define XS_BM 256
#endif
#ifndef XS_WGPC
#define XS_WGPC 1
#endif
constexpr int kBlockM = XS_BM;         // query rows per workgroup
constexpr int kBlockN = 64;            // keys per K/V block of the schedule
constexpr int kUnitKeys = 2 * kBlockN; // keys per schedule unit (a pair of blocks)
constexpr int kGroupsPerCU = XS_WGPC;  // workgroups resident per compute unit
constexpr int kHalfM = kBlockM / 2;    // query rows per workgroup of a half-height launch

// The work schedule, shared by the kernels, the merge and the host plan.
// Tiles are numbered tile = (b*H + h) * mtiles + m-tile.  Workgroup share c
// (c = 0 .. groups-1, XCD-aware: the workgroups of one XCD take consecutive
// shares) first processes the whole tiles r*groups + c for r = 0 .. dp-1 --
// in rounds, so the workgroups of an XCD stream neighbouring tiles of one head
// over the same keys together and share K/V in L2 -- and then an equal share
// of the remaining tiles' units: units u = (tile - dp*groups) * npair + pair
// (pair = key blocks 2*pair, 2*pair+1), share c owning [start(c), start(c+1))
// with start(c) = floor(c * units / groups), walked as pieces (maximal runs
// inside one tile).  A piece that is a whole tile is normalised and stored
// directly; a cut piece (only the first and the last piece of a share's
// remainder run can be cut) writes its partials into slot 2c (first) or 2c+1
// (any later piece).
struct Sched {
  long long units;  // units of the remainder tiles
  int groups, npair, dp;
  __host__ __device__ long long start(int c) const { return (long long)c * units / groups; }
  // the share that owns remainder unit u
  __host__ __device__ int owner(long long u) const {
    return (int)(((u + 1) * (long long)groups - 1) / units);
  }
};

hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t stream);

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t stream);
hipError_t launch_attn_fp8(const AttnArgs& a, hipStream_t stream);

}  // namespace xs
