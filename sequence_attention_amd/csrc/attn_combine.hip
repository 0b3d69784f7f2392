// attn_combine.hip -- merges the fp32 partial results of the query tiles that
// the work schedule cut between workgroups into the bf16 destination-ordered
// output.
//
// Each piece s of a query row holds O_s = sum_j 2^(s_j c - m_s) v_j (not
// normalised), its running max m_s (log2 units) and row sum l_s.  The row is
//   M = max_s m_s,  w_s = 2^(m_s - M),  O = sum_s w_s O_s / sum_s w_s l_s,
// the online-softmax merge of partial attention ("Move the Query, Not the
// Cache", gist.science explainer: Methodik, the Route primitive merges partial
// attention computed at the owner with an online softmax).  The pieces are
// summed in key order, so the result is deterministic.  The row's
// log-sum-exp, when asked for, is ln(2^M L) with L = sum_s w_s l_s.
#include "attn_launch.h"
#include "device_common.h"

namespace xs {

// The attention kernels store a piece's O in the register order of their
// 32x32 accumulators: per 32-row group of the tile, D/8 chunks of 64 lanes x
// 4 floats, lane L holding row L%32 and, in chunk k, the columns
// 32(k/4) + 8(k%4) + 4(L/32) .. +3 of it.  Each workgroup here reads four chunks of one
// 32-row group (one per wave, 1 KiB contiguous per piece) and merges them.
// Tiles held whole by one share of the schedule were stored by the attention
// kernel: those workgroups exit.  For a cut tile the pieces are, in key order,
// the last piece of the share that owns its first unit (slot 2c+1, or 2c if
// that share's remainder run starts exactly at the tile) and the first piece
// of every later share up to the owner of its last unit (slot 2c).
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  constexpr int CH = D / 8;                   // chunks per 32-row group
  constexpr int WPG = CH / 4;                 // workgroups per 32-row group
  constexpr int GPT = (kBlockM / 32) * WPG;   // workgroups per tile
  const Sched sch{a.units, a.groups, a.npair, a.dp};
  // only the remainder tiles can be cut: the grid covers them alone
  const int rt = blockIdx.x / GPT;  // index among the remainder tiles
  const int tile = a.dp * a.groups + rt;
  const long long u0 = (long long)rt * a.npair, u1 = u0 + a.npair - 1;
  const int c_lo = sch.owner(u0), c_hi = sch.owner(u1);
  if (c_lo == c_hi) return;
  const int mtiles = (a.S + kBlockM - 1) / kBlockM;
  const int bh = tile / mtiles;
  const int wg = blockIdx.x % GPT;
  const int g = wg / WPG;                                      // 32-row group
  const int k = (wg % WPG) * 4 + (int)(threadIdx.x >> 6);      // chunk
  const int ln = threadIdx.x & 63;
  const int r = g * 32 + (ln & 31);  // row within the tile
  const int srow = (tile - bh * mtiles) * kBlockM + r;
  if (srow >= a.S) return;
  const int d0 = (k >> 2) * 32 + (k & 3) * 8 + 4 * (ln >> 5);
  const size_t ooff = ((size_t)(g * CH + k) * 64 + ln) * 4;  // within a slot's O
  // every share holds at least one remainder unit (the plan keeps units >= groups)
  const size_t first = 2 * (size_t)c_lo + (sch.start(c_lo) < u0 ? 1 : 0);
  auto slot_of = [&](int c) { return c == c_lo ? first : 2 * (size_t)c; };

  // Pieces in groups of up to four: all loads of a group are issued before any
  // is used (the merge is bound by memory latency, not bandwidth).  Each group
  // is folded into the running (M, L, acc) with the online-softmax rescale,
  // in key order.
  float M = -INFINITY, L = 0.0f;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int c0 = c_lo; c0 <= c_hi; c0 += 4) {
    f32x2 ml[4];
    f32x4 o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = c0 + i <= c_hi ? c0 + i : c_hi;  // clamped: a repeated load, not used
      const size_t sr = slot_of(c) * kBlockM + r;
      ml[i] = *(const f32x2*)(a.ws_ml + 2 * sr);
      o[i] = *(const f32x4*)(a.ws_o + slot_of(c) * kBlockM * D + ooff);
    }
    float Mg = M;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (c0 + i <= c_hi) Mg = fmaxf(Mg, ml[i][0]);
    const float a0 = fast_exp2(M - Mg);  // 0 for the first group (M = -inf)
    L *= a0;
    acc *= a0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (c0 + i <= c_hi) {
        const float w = fast_exp2(ml[i][0] - Mg);
        L += w * ml[i][1];
        acc += w * o[i];
      }
    M = Mg;
  }
  const float inv = a.o_scale / L;
  if (a.lse && d0 == 0) a.lse[(size_t)bh * a.S + srow] = row_lse(M, L);
  const int H = a.H, T = a.T;
  const int h = bh % H, b = bh / H;
  const int p = srow / T;
  const int sp = srow - p * T;
  uint16_t* dst = (uint16_t*)a.out + ((((size_t)p * a.B + b) * T + sp) * H + h) * D + d0;
  *(u32x2*)dst = u32x2{pack_bf16(acc[0] * inv, acc[1] * inv), pack_bf16(acc[2] * inv, acc[3] * inv)};
}

template <int D>
static hipError_t launch_combine_d(const AttnArgs& a, hipStream_t stream) {
  constexpr int GPT = (kBlockM / 32) * (D / 32);  // workgroups per tile, as in the kernel
  const long long blocks = a.units / a.npair * GPT;
  if (blocks < 1 || blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  AttnArgs args = a;
  void* kargs[] = {&args};
  return hipLaunchKernel((const void*)attn_combine_kernel<D>, dim3((unsigned)blocks), dim3(256), kargs, 0,
                         stream);
}

hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t stream) {
  switch (a.D) {
    case 64:
      return launch_combine_d<64>(a, stream);
    case 128:
      return launch_combine_d<128>(a, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace xs
