// piece.h -- decoding a piece of a workgroup's chunk of the work schedule
// (attn_launch.h, Sched): shared by the bf16 and fp8 kernels.
#pragma once

#include "attn_launch.h"
#include "device_common.h"

namespace xs {

// Key blocks [jb, je) of one query tile, and the addressing its loads need.
// All members are wave-uniform.
struct PieceAddr {
  int bh, b, h, m0, jb, je;
  bool whole;        // the piece covers the tile's whole key range
  size_t head_off;   // byte offset of row 0 of (b, h) in q, k, v
  ChunkCursor kcur, vcur;
};

// Pieces of one workgroup's share of the schedule, in order: its whole tiles
// first, then the pieces of its run of remainder units.  Wave-uniform state.
struct ShareWalk {
  int chunk, round;
  long long u, uend;
  int sk_pieces;  // remainder pieces handed out so far
  __device__ void init(const Sched& s, int c) {
    chunk = c, round = 0, sk_pieces = 0;
    u = s.start(c);
    uend = s.start(c + 1);
  }
  __device__ bool more(const Sched& s) const { return round < s.dp || u < uend; }
};

// The next piece of the walk (more() must hold), for query tiles of BM rows,
// input rows of ROWB bytes (one head) and key blocks of BN keys (nblk blocks
// in all); `slot` receives the workspace slot a cut piece writes.
template <int BM, int ROWB, int BN>
__device__ __forceinline__ PieceAddr next_piece(ShareWalk& w, const Sched& sch, const AttnArgs& a,
                                                int nblk, uint32_t row_stride, int& slot) {
  const int npair = sch.npair, mtiles = (a.S + BM - 1) / BM;
  int tile, p0, p1;
  if (w.round < sch.dp) {
    tile = a.tile0 + w.round * sch.groups + w.chunk;
    p0 = 0;
    p1 = npair;
    ++w.round;
    slot = -1;
  } else {
    const int rt = (int)(w.u / npair);
    tile = a.tile0 + sch.dp * sch.groups + rt;
    p0 = (int)(w.u - (long long)rt * npair);
    const long long left = w.uend - w.u;
    p1 = left < npair - p0 ? p0 + (int)left : npair;
    w.u += p1 - p0;
    slot = 2 * w.chunk + (w.sk_pieces > 0 ? 1 : 0);
    ++w.sk_pieces;
  }
  PieceAddr pa;
  pa.bh = tile / mtiles;
  pa.m0 = (tile - pa.bh * mtiles) * BM;
  pa.h = pa.bh % a.H;
  pa.b = pa.bh / a.H;
  static_assert(kUnitKeys % (2 * BN) == 0, "a unit holds an even number of blocks");
  constexpr int BPU = kUnitKeys / BN;  // key blocks per unit
  pa.jb = BPU * p0;
  pa.je = BPU * p1 < nblk ? BPU * p1 : nblk;
  pa.whole = p0 == 0 && p1 == npair;
  pa.head_off = ((size_t)pa.b * a.batch_rows * a.H + pa.h) * ROWB;
  pa.kcur.init(pa.jb, a.chunk_rows, a.jump_rows, row_stride);
  pa.vcur.init(pa.jb, a.chunk_rows, a.jump_rows, row_stride);
  return pa;
}

}  // namespace xs
