// attn_combine.hip -- merges the fp32 partial results of a key range split
// into the bf16 destination-ordered output.
//
// Each split s of a query row holds O_s = sum_j 2^(s_j c - m_s) v_j (not
// normalised), its running max m_s (log2 units) and row sum l_s.  The row is
//   M = max_s m_s,  w_s = 2^(m_s - M),  O = sum_s w_s O_s / sum_s w_s l_s,
// the online-softmax merge of partial attention ("Move the Query, Not the
// Cache", gist.science explainer: Methodik, the Route primitive merges partial
// attention computed at the owner with an online softmax).  The splits are
// summed in a fixed order, so the result is deterministic.  The row's
// log-sum-exp, when asked for, is ln(2^M L) with L = sum_s w_s l_s.
#include "attn_launch.h"
#include "device_common.h"

namespace xs {

template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  constexpr int LPR = D / 4;             // lanes per row, 4 consecutive d each
  constexpr int RPB = 256 / LPR;         // rows per workgroup
  const size_t rows = (size_t)a.B * a.H * a.S;
  const size_t row = (size_t)blockIdx.x * RPB + threadIdx.x / LPR;
  if (row >= rows) return;
  const int d0 = (threadIdx.x % LPR) * 4;

  float M = -INFINITY;
  for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, a.ws_ml[2 * ((size_t)s * rows + row)]);
  float L = 0.0f;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s = 0; s < a.nsplit; ++s) {
    const size_t r = (size_t)s * rows + row;
    const f32x2 ml = *(const f32x2*)(a.ws_ml + 2 * r);
    const float w = fast_exp2(ml[0] - M);
    L += w * ml[1];
    acc += w * *(const f32x4*)(a.ws_o + r * D + d0);
  }
  const float inv = a.o_scale / L;
  if (a.lse && d0 == 0) a.lse[row] = row_lse(M, L);
  const int S = a.S, H = a.H, T = a.T;
  const int srow = (int)(row % S);
  const int bh = (int)(row / S);
  const int h = bh % H, b = bh / H;
  const int p = srow / T;
  const int sp = srow - p * T;
  uint16_t* dst = (uint16_t*)a.out + ((((size_t)p * a.B + b) * T + sp) * H + h) * D + d0;
  *(u32x2*)dst = u32x2{pack_bf16(acc[0] * inv, acc[1] * inv), pack_bf16(acc[2] * inv, acc[3] * inv)};
}

template <int D>
static hipError_t launch_combine_d(const AttnArgs& a, hipStream_t stream) {
  constexpr int RPB = 256 / (D / 4);
  const size_t rows = (size_t)a.B * a.H * a.S;
  const size_t blocks = (rows + RPB - 1) / RPB;
  if (blocks > 0x7fffffffULL) return hipErrorInvalidValue;
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
