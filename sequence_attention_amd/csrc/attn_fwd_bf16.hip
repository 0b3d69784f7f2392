// attn_fwd_bf16.hip -- non-causal multi-head attention forward pass over bf16
// Q/K/V for gfx950, fused with the destination-ordered epilogue.
//
// Operation (X-Stage paper, catalyzex.com abstract; gist.science explainer,
// "Zentrale Beitraege", "FlashAttention-A2A (Piggybacking)"): FlashAttention
// over the full sequence for each (batch, head) of this GPU's Ulysses share;
// the wave that owns an output tile stores it directly into the P-way buffer
// the post-attention All-to-All delivers, then moves on -- there is no separate
// communication wave and no separate relayout pass.
//
// Design (one workgroup = NW waves = BM = NW*32*QT query rows of one (b, h)):
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    each lane then owns one query column and 16 keys of every 32x32 score
//    tile, so the row max and row sum are lane-local except for one
//    permlane32 swap between the two half-waves.
//  * The transposed probabilities P^T leave the accumulator already in the
//    B-operand layout of O^T += V^T P^T (the key order inside a k-step is
//    permuted identically on both operands), so P never goes through LDS.
//  * K/V tiles of BN = 64 keys are double buffered in LDS and filled with
//    direct-to-LDS 16-byte loads (no VGPR round trip).  K rows are XOR
//    swizzled for conflict-free ds_read_b128 of the A operand; V rows are
//    swizzled for ds_read_b64_tr_b16, which delivers V^T fragments directly.
//  * Online softmax in base 2: p = 2^(s*c - m) with c = scale*log2(e) folded
//    into one FMA per score.  The running max m is only moved (and O, l
//    rescaled) when a block's max exceeds it by more than 2^8, so p <= 256
//    and the rescale is a rare wave-uniform branch.
//  * Epilogue: O/l rounded to bf16 and stored per query row at its
//    destination-slice offset (p = s / T, s' = s - p*T).  Tile shapes and the
//    reduction order never depend on P; only the store address does.
#include "attn_launch.h"
#include "device_common.h"

namespace xs {

template <int D_, int QT_, int NW_>
struct Bf16Cfg {
  static constexpr int D = D_;
  static constexpr int QT = QT_;         // 32-query sub-tiles per wave
  static constexpr int NW = NW_;         // waves per workgroup
  static constexpr int BN = 64;          // keys per K/V block
  static constexpr int QW = 32 * QT;     // queries per wave
  static constexpr int BM = QW * NW;     // queries per workgroup
  static constexpr int CH = D / 8;       // 16-byte chunks per K/V row
  static constexpr int ROWB = D * 2;     // bytes per K/V row in LDS
  static constexpr int TILE = BN * ROWB; // bytes per K or V tile
  static constexpr int LOADS = TILE / 1024;
  static constexpr int LPW = LOADS / NW; // 1 KiB direct loads per wave per tile
  static constexpr int KS = D / 16;      // k-steps of QK^T
  static constexpr int DT = D / 32;      // 32-row d tiles of O^T
  static constexpr int NT = BN / 32;     // 32-key tiles per block
  static constexpr int THREADS = 64 * NW;
  static_assert(LOADS % NW == 0 && LOADS >= NW, "tile loads must split evenly over waves");
  static constexpr float TAU = 8.0f;     // lazy-rescale threshold (log2 units)
};

// Per-lane byte offsets (relative to the block's first key row) of the
// 16-byte chunks this lane moves for one K (SWZ_V = false) or V (SWZ_V = true)
// tile: LDS chunk position pos holds global chunk (pos % CH) ^ swizzle(row).
template <class C, bool SWZ_V>
__device__ __forceinline__ void tile_offsets(uint32_t row_stride, int wave, int lane,
                                             uint32_t (&voff)[C::LPW]) {
#pragma unroll
  for (int i = 0; i < C::LPW; ++i) {
    const int pos = (wave * C::LPW + i) * 64 + lane;
    const int row = pos / C::CH;
    const int swz = SWZ_V ? ((2 * row) & (C::CH - 1)) : (row & (C::CH - 1));
    const int chunk = (pos % C::CH) ^ swz;
    voff[i] = (uint32_t)row * row_stride + (uint32_t)chunk * 16u;
  }
}

// Fill one K or V tile of BN rows starting at key kv0 with direct-to-LDS
// buffer loads.  The buffer resource ends after row S-1, so rows past the end
// of the sequence read as zeros (their scores are masked).
template <class C>
__device__ __forceinline__ void load_tile(const uint8_t* head_base, uint32_t row_stride, int kv0,
                                          int S, const uint8_t XS_LDS* dst,
                                          const uint32_t (&voff)[C::LPW], int wave) {
  const u32x4 rsrc = make_rsrc(head_base + (size_t)kv0 * row_stride,
                               (uint32_t)(S - kv0 - 1) * row_stride + (uint32_t)C::ROWB);
  const uint32_t base = lds_addr(dst) + (uint32_t)(wave * C::LPW) * 1024u;
#pragma unroll
  for (int i = 0; i < C::LPW; ++i) load_lds_b128(rsrc, voff[i], base + i * 1024u);
}

template <class C>
struct Bf16State {
  f32x16 o[C::QT][C::DT];
  float m[C::QT];
  float l[C::QT];
  u32x4 qf[C::QT][C::KS];
};

// One K/V block: scores, online softmax, P V.
template <class C, bool MASK>
__device__ __forceinline__ void block_step(Bf16State<C>& st, const uint8_t XS_LDS* sK,
                                           const uint8_t XS_LDS* sV, int kv0, int S, float c,
                                           int lane) {
  constexpr int QT = C::QT, NT = C::NT, KS = C::KS, DT = C::DT, CH = C::CH, ROWB = C::ROWB;
  const int hi = lane >> 5;

  // ---- S^T = K Q^T
  f32x16 s[NT][QT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) s[nt][qt] = f32x16{};
  const uint8_t XS_LDS* krow = sK + (lane & 31) * ROWB;
  const int ksw = lane & (CH - 1);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const u32x4 kf = lds_read_b128(krow + nt * 32 * ROWB + (((2 * ks + hi) ^ ksw) << 4));
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) s[nt][qt] = mfma_bf16(kf, st.qf[qt][ks], s[nt][qt]);
    }
  }

  // keep the phases apart so the V fragments are not all hoisted into registers
  // next to the live scores
  __builtin_amdgcn_sched_barrier(0);

  // ---- online softmax (lane owns query column lane%32 of every tile)
  if (MASK) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kv0 + nt * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
        if (key >= S)
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) s[nt][qt][r] = -INFINITY;
      }
  }
  float mnew[QT];
  bool need_any = false;
  bool need[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    float mx = s[0][qt][0];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[nt][qt][r]);
    mx = max_halves(mx) * c;
    mnew[qt] = fmaxf(st.m[qt], mx);
    need[qt] = mnew[qt] > st.m[qt] + C::TAU;
    need_any |= need[qt];
  }
  if (__builtin_amdgcn_ballot_w64(need_any)) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float alpha = need[qt] ? fast_exp2(st.m[qt] - mnew[qt]) : 1.0f;
      st.m[qt] = need[qt] ? mnew[qt] : st.m[qt];
      st.l[qt] *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.o[qt][dt][r] *= alpha;
    }
  }
  u32x4 pb[QT][NT][2];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float neg_m = -st.m[qt];
    float lsum = 0.0f;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = fast_exp2(__builtin_fmaf(s[nt][qt][r], c, neg_m));
        if (MASK) {
          const int key = kv0 + nt * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
          p[r] = key < S ? p[r] : 0.0f;
        }
        lsum += p[r];
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
        pb[qt][nt][h] = u32x4{pack_bf16(p[8 * h + 0], p[8 * h + 1]), pack_bf16(p[8 * h + 2], p[8 * h + 3]),
                              pack_bf16(p[8 * h + 4], p[8 * h + 5]), pack_bf16(p[8 * h + 6], p[8 * h + 7])};
    }
    st.l[qt] += lsum;
  }

  __builtin_amdgcn_sched_barrier(0);

  // ---- O^T += V^T P^T   (V^T fragments via LDS transpose reads)
  const int g = lane >> 4, L = lane & 15;
  const int vrow = 4 * (g >> 1) + (L >> 2);  // row within an 8-row group
  const int vsw = (2 * vrow) & (CH - 1);
  const uint8_t XS_LDS* vbase = sV + vrow * ROWB + 8 * (L & 1);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int chunk = (dt * 4 + 2 * (g & 1) + ((L & 3) >> 1)) ^ vsw;
        const uint8_t XS_LDS* p0 = vbase + (nt * 32 + 16 * h) * ROWB + (chunk << 4);
        const u32x2 lo = lds_read_tr16(p0);
        const u32x2 up = lds_read_tr16(p0 + 8 * ROWB);
        const u32x4 vf = u32x4{lo[0], lo[1], up[0], up[1]};
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) st.o[qt][dt] = mfma_bf16(vf, pb[qt][nt][h], st.o[qt][dt]);
      }
}

template <class C>
__global__ __launch_bounds__(C::THREADS, 1) void attn_fwd_bf16_kernel(AttnArgs a) {
  constexpr int QT = C::QT, KS = C::KS, DT = C::DT, BM = C::BM, BN = C::BN;
  // [stage][K tile | V tile], two stages
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * C::TILE];
  uint8_t XS_LDS* const lds = (uint8_t XS_LDS*)smem;

  const int S = a.S, H = a.H;
  const int mtiles = (S + BM - 1) / BM;
  const int ntiles = a.B * H * mtiles;
  const int tile = xcd_tile(blockIdx.x, ntiles);
  const int mt = tile % mtiles;
  const int bh = tile / mtiles;
  const int h = bh % H, b = bh / H;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int m0 = mt * BM;

  const uint32_t row_stride = (uint32_t)H * C::ROWB;  // bytes between consecutive rows
  const size_t head_off = ((size_t)b * S * H + h) * C::ROWB;
  const uint8_t* kbase = (const uint8_t*)a.k + head_off;
  const uint8_t* vbase = (const uint8_t*)a.v + head_off;
  uint32_t koff[C::LPW], voff[C::LPW];
  tile_offsets<C, false>(row_stride, wave, lane, koff);
  tile_offsets<C, true>(row_stride, wave, lane, voff);

  // first K/V block in flight while the queries load
  load_tile<C>(kbase, row_stride, 0, S, lds, koff, wave);
  load_tile<C>(vbase, row_stride, 0, S, lds + C::TILE, voff, wave);

  Bf16State<C> st;
  const uint32_t qflip = a.neg ? 0x80008000u : 0u;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    int qrow = m0 + wave * C::QW + qt * 32 + (lane & 31);
    qrow = qrow < S ? qrow : S - 1;
    const uint8_t* qp = (const uint8_t*)a.q + head_off + (size_t)qrow * row_stride + (lane >> 5) * 16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 t = *(const u32x4*)(qp + ks * 32);
      st.qf[qt][ks] = t ^ qflip;
    }
    st.m[qt] = -INFINITY;
    st.l[qt] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) st.o[qt][dt] = f32x16{};
  }

  const float c = a.c;
  const int nblk = (S + BN - 1) / BN;
  const int nfull = S / BN;  // blocks with no key past the end of the sequence
  for (int j = 0; j < nblk; ++j) {
    // block j's tiles (issued one block earlier) are complete in every wave, and
    // every wave is done reading the stage block j+1 is about to overwrite
    wait_vmcnt<0>();
    __syncthreads();
    uint8_t XS_LDS* const cur = lds + (j & 1) * 2 * C::TILE;
    if (j + 1 < nblk) {
      uint8_t XS_LDS* const nxt = lds + ((j + 1) & 1) * 2 * C::TILE;
      load_tile<C>(kbase, row_stride, (j + 1) * BN, S, nxt, koff, wave);
      load_tile<C>(vbase, row_stride, (j + 1) * BN, S, nxt + C::TILE, voff, wave);
    }
    if (j < nfull)
      block_step<C, false>(st, cur, cur + C::TILE, j * BN, S, c, lane);
    else
      block_step<C, true>(st, cur, cur + C::TILE, j * BN, S, c, lane);
  }

  // ---- epilogue: normalise, round to bf16, store into the destination slice
  const int T = a.T, B = a.B;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float inv = a.o_scale / sum_halves(st.l[qt]);
    const int srow = m0 + wave * C::QW + qt * 32 + (lane & 31);
    if (srow < S) {
      const int p = srow / T;
      const int sp = srow - p * T;
      uint16_t* orow = (uint16_t*)a.out + ((((size_t)p * B + b) * T + sp) * H + h) * C::D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d0 = dt * 32 + r4 * 8 + 4 * (lane >> 5);
          const f32x16& o = st.o[qt][dt];
          u32x2 w = {pack_bf16(o[4 * r4 + 0] * inv, o[4 * r4 + 1] * inv),
                     pack_bf16(o[4 * r4 + 2] * inv, o[4 * r4 + 3] * inv)};
          *(u32x2*)(orow + d0) = w;
        }
    }
  }
}

template <int D>
static hipError_t launch_d(const AttnArgs& a, hipStream_t stream) {
  using C = Bf16Cfg<D, 1, 8>;
  const int mtiles = (a.S + C::BM - 1) / C::BM;
  const long long ntiles = (long long)a.B * a.H * mtiles;
  if (ntiles > 0x7fffffffLL) return hipErrorInvalidValue;
  AttnArgs args = a;
  void* kargs[] = {&args};
  return hipLaunchKernel((const void*)attn_fwd_bf16_kernel<C>, dim3((unsigned)ntiles), dim3(C::THREADS),
                         kargs, 0, stream);
}

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t stream) {
  switch (a.D) {
    case 64:
      return launch_d<64>(a, stream);
    case 128:
      return launch_d<128>(a, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace xs
