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

// The piece that starts at unit u of a chunk ending at uend, for query tiles of
// BM rows and input rows of ROWB bytes (one head).
template <int BM, int ROWB>
__device__ __forceinline__ PieceAddr decode_piece(const AttnArgs& a, long long u, long long uend,
                                                  int nblk, uint32_t row_stride) {
  const int npair = a.npair, mtiles = (a.S + BM - 1) / BM;
  const int tile = (int)(u / npair);
  const int p0 = (int)(u - (long long)tile * npair);
  const long long left = uend - u;
  const int p1 = left < npair - p0 ? p0 + (int)left : npair;
  PieceAddr pa;
  pa.bh = tile / mtiles;
  pa.m0 = (tile - pa.bh * mtiles) * BM;
  pa.h = pa.bh % a.H;
  pa.b = pa.bh / a.H;
  pa.jb = 2 * p0;
  pa.je = 2 * p1 < nblk ? 2 * p1 : nblk;
  pa.whole = p0 == 0 && p1 == npair;
  pa.head_off = ((size_t)pa.b * a.batch_rows * a.H + pa.h) * ROWB;
  pa.kcur.init(pa.jb, a.chunk_rows, a.jump_rows, row_stride);
  pa.vcur.init(pa.jb, a.chunk_rows, a.jump_rows, row_stride);
  return pa;
}

// Units (key-block pairs) a piece covers.
__device__ __forceinline__ int piece_units(const PieceAddr& pa) { return (pa.je - pa.jb + 1) / 2; }

}  // namespace xs
