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
// Design (one workgroup = 8 waves, two per SIMD; a wave owns 32 query rows;
// BM = 256 rows of one (b, h) per workgroup, one workgroup per CU):
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    each lane then owns one query column and 16 keys of every 32x32 score
//    tile, so the row max and row sum are lane-local except for one
//    permlane32 swap between the two half-waves.
//  * The transposed probabilities P^T leave the accumulator already in the
//    B-operand layout of O^T += V^T P^T (the key order inside a k-step is
//    permuted identically on both operands), so P never goes through LDS.
//  * K/V tiles of BN = 64 keys stream through a four-stage LDS ring (128 KiB
//    for D = 128), filled with direct-to-LDS 16-byte buffer loads (no VGPR
//    round trip) issued two blocks ahead, with one barrier per two blocks.
//    K rows are XOR swizzled for conflict-free ds_read_b128 of the A operand;
//    V rows are swizzled for ds_read_b64_tr_b16, which delivers V^T fragments
//    directly.
//  * Software pipeline inside the wave:
//      step 1: QK^T of block j+1 (MFMA)  ||  exp/sum/convert of most keys of block j
//      step 2: P V of block j (MFMA)     ||  exp/sum/convert of its other keys
//    so the matrix core and the vector ALU work on different blocks at once;
//    each pair's conversion runs one micro-step after its exponentials.
//  * Online softmax in base 2: p = 2^(s*c - m), c = scale*log2(e) folded into
//    one FMA per score.  First pass over a piece: m is the exact max of the
//    piece's first block and stays there -- no checks, no rescale in the key
//    loop; later probabilities may exceed 1, which floating point carries
//    without loss.  If afterwards any lane's part of a row sum is above 2^40
//    (or not finite), the workgroup runs the piece again with the lazy
//    rescale: the running max is taken exactly for the piece's first and last
//    blocks only; the other blocks' probabilities are computed with the
//    current m and checked: when a lane's sum of a block's new p exceeds
//    2^TAU (as any single p above 2^TAU makes it), the block's exact max is
//    taken, m moves if that max exceeds it by more than TAU (log2 units), O is
//    rescaled (a rare wave-uniform branch) and the block's p are recomputed.
//    The row sum adds the fp32 p before their rounding to bf16 (plain adds:
//    the vector ALU is the scarce unit here).
//  * Epilogue: O/l rounded to bf16 and stored per query row at its
//    destination-slice offset (p = s / T, s' = s - p*T).  Tile shapes and the
//    reduction order never depend on P; only the store address does.
#include "attn_launch.h"
#include "device_common.h"
#include "piece.h"

#ifndef XS_QT
#define XS_QT 1
#endif
#ifndef XS_NW
#define XS_NW 8
#endif
#ifndef XS_BN
#define XS_BN 64
#endif

namespace xs {

template <int D_, int QT_, int NW_, int BN_>
struct Bf16Cfg {
  static constexpr int D = D_;
  static constexpr int QT = QT_;         // 32-query sub-tiles per wave
  static constexpr int NW = NW_;         // waves per workgroup
  static constexpr int BN = BN_;         // keys per K/V block
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
  static constexpr int STAGES = 4;       // LDS ring depth for K and for V
  static constexpr float TAU = 8.0f;     // lazy-rescale threshold (log2 units)
  static constexpr float PMAX = 256.0f;  // 2^TAU: the largest probability kept
  static_assert(LOADS % NW == 0 && LOADS >= NW, "tile loads must split evenly over waves");
};

// XOR swizzle of the 16-byte chunk index of V row `row`.  A ds_read_b64_tr_b16
// of a V^T fragment touches 8 rows x 4 chunks and is served one half-wave at a
// time (4 rows x 4 chunks = 256 bytes): XOR-ing the chunk with 4*(row%4) (D=128,
// one row per 256-byte bank line) or 4*((row/2)%2) (D=64, two rows per line)
// puts the 16 chunks of each half-wave on 16 different bank groups.
template <class C>
__device__ __forceinline__ int vswz(int row) {
  constexpr int RPL = 256 / C::ROWB;  // rows per 256-byte bank line
  return 4 * ((row / RPL) & (C::CH / 4 - 1));
}

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
    const int swz = SWZ_V ? vswz<C>(row) : (row & (C::CH - 1));
    const int chunk = (pos % C::CH) ^ swz;
    voff[i] = (uint32_t)row * row_stride + (uint32_t)chunk * 16u;
  }
}

// Fill one K or V tile of BN rows starting at key kv0 (rows kv0.. are `extra`
// bytes further in the chunk input layout) with direct-to-LDS buffer loads.
// The buffer resource ends after row S-1, so rows past the end of the sequence
// read as zeros (their scores are masked).
template <class C>
__device__ __forceinline__ void load_tile(const uint8_t* head_base, uint32_t row_stride, int kv0,
                                          size_t extra, int S, const uint8_t XS_LDS* dst,
                                          const uint32_t (&voff)[C::LPW], int wave) {
  const u32x4 rsrc = make_rsrc(head_base + (size_t)kv0 * row_stride + extra,
                               (uint32_t)(S - kv0 - 1) * row_stride + (uint32_t)C::ROWB);
  const uint32_t base = lds_addr(dst) + (uint32_t)(wave * C::LPW) * 1024u;
#pragma unroll
  for (int i = 0; i < C::LPW; ++i) load_lds_b128(rsrc, voff[i], base + i * 1024u);
}

template <class C>
struct Scores {
  f32x16 s[C::NT][C::QT];  // S^T tiles: [32-key tile][query sub-tile]
};

template <class C>
struct Bf16State {
  f32x16 o[C::QT][C::DT];     // O^T accumulators: lane owns query lane%32 of each sub-tile
  u32x4 qf[C::QT][C::KS];     // Q^T B-operand fragments
  u32x4 pb[C::QT][2 * C::NT]; // bf16 probabilities, P^T B-operand fragment F = keys 16F..16F+15
  float m[C::QT];             // running max of s*c (log2 units), shared by both half-waves
  float l[C::QT];             // lane-local part of the running sum of p
  float lh[C::QT];            // l through the probabilities of the first half of a block's keys
  float alpha[C::QT];         // pending rescale of O (applied before the next P V)
  bool rescale;               // wave-uniform: alpha differs from 1 somewhere
};

// ---- step-1 MFMA work: S^T = K_j Q^T
template <class C>
__device__ __forceinline__ void qk_block(Scores<C>& sc, const Bf16State<C>& st,
                                         const uint8_t XS_LDS* sK, int lane) {
  constexpr int QT = C::QT, NT = C::NT, KS = C::KS, CH = C::CH, ROWB = C::ROWB;
  const int ln = opaque(lane);
  const int hi = ln >> 5;
  const uint8_t XS_LDS* krow = sK + (ln & 31) * ROWB;
  const int ksw = ln & (CH - 1);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const u32x4 kf = lds_read_b128(krow + nt * 32 * ROWB + (((2 * ks + hi) ^ ksw) << 4));
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
        sc.s[nt][qt] = mfma_bf16(kf, st.qf[qt][ks], ks == 0 ? f32x16{} : sc.s[nt][qt]);
    }
  }
}

// O^T *= alpha, one 32x32 tile at a time (the scheduling barriers keep the
// tiles apart, so the rare rescale does not raise the register pressure).
template <class C>
__device__ __forceinline__ void rescale_o(Bf16State<C>& st) {
#pragma unroll
  for (int qt = 0; qt < C::QT; ++qt) {
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      st.o[qt][dt] *= st.alpha[qt];
      __builtin_amdgcn_sched_barrier(0);
    }
    st.alpha[qt] = 1.0f;
  }
  st.rescale = false;
}

// Keys at or past S (only in the last, partial block) get score -inf.
template <class C>
__device__ __forceinline__ void mask_tail(Scores<C>& sc, int kv0, int S, int lane) {
  const int hi = lane >> 5;
#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kv0 + nt * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
      if (key >= S)
#pragma unroll
        for (int qt = 0; qt < C::QT; ++qt) sc.s[nt][qt][r] = -INFINITY;
    }
}

// ---- row max of a scored block, lazy move of the running max (piece ends and
// the rare overflow path); returns whether the max moved
template <class C>
__device__ __forceinline__ bool softmax_max(Bf16State<C>& st, const Scores<C>& sc, float c) {
  constexpr int QT = C::QT, NT = C::NT;
  bool need[QT], any = false;
  float mnew[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    float mx = sc.s[0][qt][0];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc.s[nt][qt][r]);
    mnew[qt] = max_halves(mx) * c;  // finite: every block holds a valid key
    need[qt] = mnew[qt] > st.m[qt] + C::TAU;
    any |= need[qt];
  }
  if (__builtin_amdgcn_ballot_w64(any)) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float a = need[qt] ? fast_exp2(st.m[qt] - mnew[qt]) : 1.0f;  // 0 when m = -inf
      st.m[qt] = need[qt] ? mnew[qt] : st.m[qt];
      st.l[qt] *= a;
      st.alpha[qt] *= a;
    }
    st.rescale = true;
    return true;
  }
  return false;
}

// ---- step-1 VALU work: p = 2^(s c - m) -> bf16 P^T fragments, row sums
template <class C>
__device__ __forceinline__ void softmax_exp(Bf16State<C>& st, const Scores<C>& sc, float c) {
  constexpr int QT = C::QT, NT = C::NT;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float neg_m = -st.m[qt];
    float lsum = st.l[qt];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p0 = fast_exp2(__builtin_fmaf(sc.s[nt][qt][8 * h + 2 * i], c, neg_m));
          const float p1 = fast_exp2(__builtin_fmaf(sc.s[nt][qt][8 * h + 2 * i + 1], c, neg_m));
          w[i] = pack_bf16(p0, p1);
          lsum += p0;
          lsum += p1;
        }
        st.pb[qt][2 * nt + h] = u32x4{w[0], w[1], w[2], w[3]};
      }
    st.l[qt] = lsum;
  }
}

// LDS fragments are read LEAD micro-steps before their MFMA (2 measured 0.5 %
// faster than 3 on the video share with the rescale-free first pass; 4 and 5 the same)
#ifndef XS_LEAD
#define XS_LEAD 2
#endif

// ---- The two steps of the software pipeline, written as fixed sequences of
// micro-steps separated by scheduling barriers: each micro-step reads the LDS
// fragment LEAD positions ahead, issues the MFMA that uses the fragment read
// LEAD micro-steps earlier, and does a slice of the softmax work, so LDS
// latency and vector work hide under the matrix core.  The exponentials of a
// block are split between the two steps (those the first half of its P V
// needs, and at D = 128 some more, under the next block's QK^T; the rest under
// the first half of this block's P V) so that neither step is bound by the
// vector ALU.  LDS addresses are per-lane offsets computed once plus
// immediates (the ring stage is a template argument).

// Per-lane LDS byte offsets of the fragments, relative to a tile's start.
template <class C>
struct LdsOffs {
  uint32_t k[C::KS];  // K fragment of k-step ks (row lane%32, chunk 2ks + lane/32)
  uint32_t v[C::DT];  // first V^T transpose read of d-tile dt (rows 0..7 group), V region
};

template <class C>
__device__ __forceinline__ LdsOffs<C> lds_offsets(int lane) {
  LdsOffs<C> o;
  const int hi = lane >> 5, ksw = lane & (C::CH - 1);
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks)
    o.k[ks] = (uint32_t)((lane & 31) * C::ROWB + (((2 * ks + hi) ^ ksw) << 4));
  const int g = lane >> 4, L = lane & 15;
  const int vrow = 4 * (g >> 1) + (L >> 2);
  const int vsw = vswz<C>(vrow);  // rows of a fragment differ from vrow by multiples of 8
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) {
    const int chunk = (dt * 4 + 2 * (g & 1) + ((L & 3) >> 1)) ^ vsw;
    o.v[dt] = (uint32_t)(C::STAGES * C::TILE + vrow * C::ROWB + 8 * (L & 1) + (chunk << 4));
  }
  return o;
}

// The probabilities of one score pair in two halves, a micro-step apart, so
// the conversion never waits on the transcendental unit's latency:
//  exp_pair2: p = 2^(s c - m) of pair idx (0 .. 8 NT - 1: registers 2(idx%8),
//             2(idx%8)+1 of 32-key tile idx/8) of query sub-tile qt;
//  pack_sum:  the pair rounded to bf16 (word idx%4 of P^T fragment idx/4);
//             its fp32 values added to the row sum.
// Both are pinned to the micro-step they are issued in.
template <class C>
__device__ __forceinline__ f32x2 exp_pair2(const Scores<C>& cur, int qt, int idx, float c,
                                           float neg_m) {
  const int nt = idx / 8, e = idx % 8;
  float p0 = fast_exp2(__builtin_fmaf(cur.s[nt][qt][2 * e], c, neg_m));
  float p1 = fast_exp2(__builtin_fmaf(cur.s[nt][qt][2 * e + 1], c, neg_m));
  pin(p0);
  pin(p1);
  return f32x2{p0, p1};
}

__device__ __forceinline__ uint32_t pack_sum(f32x2 p, float& lsum) {
  uint32_t pk = pack_bf16(p[0], p[1]);
  lsum += p[0];
  lsum += p[1];
  pin(pk);
  pin(lsum);
  return pk;
}

#ifndef XS_NE1
#define XS_NE1 0
#endif

// The score pairs of a block in the order the pipeline computes them: first
// those of the first half of the block's keys (P^T fragments F < NT, used by
// the first half of P V) for every sub-tile, then those of the second half.
// Step 1 computes pairs 0 .. NE1-1, step 2 the rest under its first half.
// At D = 128 step 1 takes three quarters of the pairs (measured 0.4 % faster
// than an even split on the video share); at D = 64 the two splits measure
// the same and the even one is kept.
template <class C>
struct PairOrder {
  static constexpr int HP = 4 * C::NT * C::QT;  // pairs per half
  static constexpr int NP = 2 * HP;
  static constexpr int NE1 = XS_NE1 > 0 && XS_NE1 <= NP && XS_NE1 >= HP ? XS_NE1
                             : C::D == 128                                ? 3 * HP / 2
                                                                          : HP;
  static constexpr int qt(int k) { return (k % HP) / (4 * C::NT); }
  static constexpr int idx(int k) { return (k / HP) * 4 * C::NT + k % (4 * C::NT); }
  // pair k is sub-tile qt(k)'s last pair of the first half of the keys
  static constexpr bool last_of_first_half(int k) { return k < HP && (k + 1) % (4 * C::NT) == 0; }
};

// Step 1: S^T of the next block from K stage KST || the first NE1 probability
// pairs of the current block.  Each K fragment feeds the QT query sub-tiles.
template <class C, int KST, bool CHECK>
__device__ __forceinline__ void step1(Scores<C>& nxt, const Scores<C>& cur, Bf16State<C>& st,
                                      const uint8_t XS_LDS* lds, const LdsOffs<C>& off, float c) {
  using PO = PairOrder<C>;
  constexpr int QT = C::QT, NT = C::NT, KS = C::KS, ROWB = C::ROWB;
  constexpr int NF = KS * NT;
  constexpr int LEAD = XS_LEAD < NF ? XS_LEAD : NF;
  constexpr int R = LEAD + 1;
  constexpr int NE = PO::NE1;
  const uint8_t XS_LDS* kb = lds + KST * C::TILE;
  auto kread = [&](int f) { return lds_read_b128(kb + off.k[f / NT] + (f % NT) * 32 * ROWB); };
  float neg_m[QT], lsum[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    neg_m[qt] = -st.m[qt];
    lsum[qt] = st.l[qt];
  }
  u32x4 kf[R];
  f32x2 pe[NE];
#pragma unroll
  for (int f = 0; f < LEAD; ++f) kf[f] = kread(f);
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    if (f + LEAD < NF) kf[(f + LEAD) % R] = kread(f + LEAD);
    const int ks = f / NT, nt = f % NT;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
      nxt.s[nt][qt] = mfma_bf16(kf[f % R], st.qf[qt][ks], ks == 0 ? f32x16{} : nxt.s[nt][qt]);
    // the first NE pairs, spread evenly over the NF micro-steps: packed one
    // micro-step after their exponentials
#pragma unroll
    for (int k = 0; k < NE; ++k)
      if (f > 0 && k * NF / NE == f - 1) {
        const int qt = PO::qt(k), idx = PO::idx(k);
        st.pb[qt][idx / 4][idx % 4] = pack_sum(pe[k], lsum[qt]);
        if (CHECK && PO::last_of_first_half(k)) st.lh[qt] = lsum[qt];
      }
#pragma unroll
    for (int k = 0; k < NE; ++k)
      if (k * NF / NE == f) pe[k] = exp_pair2<C>(cur, PO::qt(k), PO::idx(k), c, neg_m[PO::qt(k)]);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int k = 0; k < NE; ++k)
    if (k * NF / NE == NF - 1) {
      const int qt = PO::qt(k), idx = PO::idx(k);
      st.pb[qt][idx / 4][idx % 4] = pack_sum(pe[k], lsum[qt]);
      if (CHECK && PO::last_of_first_half(k)) st.lh[qt] = lsum[qt];
    }
  // Overflow check of the pairs just computed (the running max was not taken
  // for this block): a lane whose new probabilities sum to more than 2^TAU may
  // hold one above 2^TAU (any one above it makes the sum exceed it).  Then the
  // block's exact max is taken; if the running max moves, the O rescale is left
  // pending for step 2 and these pairs are recomputed with the new max.
  bool over = false;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) over |= CHECK && !(lsum[qt] - st.l[qt] <= C::PMAX);
  if (CHECK && __builtin_amdgcn_ballot_w64(over)) {
    if (softmax_max<C>(st, cur, c)) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) lsum[qt] = st.l[qt];
#pragma unroll
      for (int k = 0; k < NE; ++k) {
        const int qt = PO::qt(k), idx = PO::idx(k);
        const f32x2 p = exp_pair2<C>(cur, qt, idx, c, -st.m[qt]);
        st.pb[qt][idx / 4][idx % 4] = pack_sum(p, lsum[qt]);
        if (PO::last_of_first_half(k)) st.lh[qt] = lsum[qt];
      }
    }
  }
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    st.l[qt] = lsum[qt];
#pragma unroll
    for (int F = 0; F < 2 * NT; ++F) keep(st.pb[qt][F]);
  }
}

// Step 2: O^T = alpha O^T + V^T P^T from V stage VST; under the first half
// (the first half of the block's keys) the remaining probability pairs, then
// their overflow check before the second half uses them.
template <class C, int VST, bool CHECK>
__device__ __forceinline__ void step2(Bf16State<C>& st, const Scores<C>& cur,
                                      const uint8_t XS_LDS* lds, const LdsOffs<C>& off, float c) {
  using PO = PairOrder<C>;
  constexpr int QT = C::QT, NT = C::NT, DT = C::DT, ROWB = C::ROWB;
  constexpr int NF = 2 * NT * DT;          // V fragments F-major: keys 16F..16F+15
  constexpr int HALF = NF / 2;
  constexpr int LEAD = XS_LEAD < NF ? XS_LEAD : NF;
  constexpr int R = LEAD + 1;
  constexpr int NE = PO::NP - PO::NE1;     // pairs left for this step
  if (CHECK && st.rescale) rescale_o<C>(st);
  const uint8_t XS_LDS* vb = lds + VST * C::TILE;  // off.v holds the V region's base
  auto vaddr = [&](int f) { return vb + off.v[f % DT] + (f / DT) * 16 * ROWB; };
  float neg_m[QT], lsum[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    neg_m[qt] = -st.m[qt];
    lsum[qt] = st.l[qt];
  }
  u32x2 vlo[R], vhi[R];
  f32x2 pe[NE > 0 ? NE : 1];
#pragma unroll
  for (int f = 0; f < LEAD; ++f) {
    vlo[f] = lds_read_tr16(vaddr(f));
    vhi[f] = lds_read_tr16(vaddr(f) + 8 * ROWB);
  }
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    if (f + LEAD < NF) {
      vlo[(f + LEAD) % R] = lds_read_tr16(vaddr(f + LEAD));
      vhi[(f + LEAD) % R] = lds_read_tr16(vaddr(f + LEAD) + 8 * ROWB);
    }
    // pack the pairs whose exponentials the previous micro-step issued (before
    // this micro-step's MFMA, which may need them)
#pragma unroll
    for (int k = 0; k < NE; ++k)
      if (f > 0 && f <= HALF && k * HALF / NE == f - 1) {
        const int qt = PO::qt(PO::NE1 + k), idx = PO::idx(PO::NE1 + k);
        st.pb[qt][idx / 4][idx % 4] = pack_sum(pe[k], lsum[qt]);
      }
    if (CHECK && f == HALF) {
      // Overflow check of this step's pairs, as in step 1.  The first half of
      // the block is already weighted into O: if the running max moves, O and
      // the sum through that half are rescaled now and the second half's pairs
      // (those of step 1 too) are recomputed with the new max.
      bool over = false;
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) over |= !(lsum[qt] - st.l[qt] <= C::PMAX);
      if (__builtin_amdgcn_ballot_w64(over)) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) st.l[qt] = st.lh[qt];  // the sum O holds
        if (softmax_max<C>(st, cur, c)) {
          rescale_o<C>(st);
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) lsum[qt] = st.l[qt];
#pragma unroll
          for (int k = PO::HP; k < PO::NP; ++k) {
            const int qt = PO::qt(k), idx = PO::idx(k);
            const f32x2 p = exp_pair2<C>(cur, qt, idx, c, -st.m[qt]);
            st.pb[qt][idx / 4][idx % 4] = pack_sum(p, lsum[qt]);
          }
        }
      }
    }
    const int F = f / DT, dt = f % DT;
    const u32x4 vf = u32x4{vlo[f % R][0], vlo[f % R][1], vhi[f % R][0], vhi[f % R][1]};
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) st.o[qt][dt] = mfma_bf16(vf, st.pb[qt][F], st.o[qt][dt]);
    if (f < HALF) {
#pragma unroll
      for (int k = 0; k < NE; ++k)
        if (k * HALF / NE == f) {
          const int qt = PO::qt(PO::NE1 + k), idx = PO::idx(PO::NE1 + k);
          pe[k] = exp_pair2<C>(cur, qt, idx, c, neg_m[qt]);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) st.l[qt] = lsum[qt];
}

// O^T = alpha O^T + V^T P^T of the last block of a piece from the V stage at
// byte offset stage_off (no next block to overlap with: its probabilities are
// complete).
template <class C, bool CHECK>
__device__ __forceinline__ void pv_only(Bf16State<C>& st, const uint8_t XS_LDS* lds,
                                        const LdsOffs<C>& off, uint32_t stage_off) {
  constexpr int QT = C::QT, DT = C::DT, ROWB = C::ROWB;
  constexpr int NF = 2 * C::NT * DT;
  constexpr int LEAD = XS_LEAD < NF ? XS_LEAD : NF;
  constexpr int R = LEAD + 1;
  if (CHECK && st.rescale) rescale_o<C>(st);
  const uint8_t XS_LDS* vb = lds + stage_off;
  auto vaddr = [&](int f) { return vb + off.v[f % DT] + (f / DT) * 16 * ROWB; };
  u32x2 vlo[R], vhi[R];
#pragma unroll
  for (int f = 0; f < LEAD; ++f) {
    vlo[f] = lds_read_tr16(vaddr(f));
    vhi[f] = lds_read_tr16(vaddr(f) + 8 * ROWB);
  }
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    if (f + LEAD < NF) {
      vlo[(f + LEAD) % R] = lds_read_tr16(vaddr(f + LEAD));
      vhi[(f + LEAD) % R] = lds_read_tr16(vaddr(f + LEAD) + 8 * ROWB);
    }
    const u32x4 vf = u32x4{vlo[f % R][0], vlo[f % R][1], vhi[f % R][0], vhi[f % R][1]};
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) st.o[qt][f % DT] = mfma_bf16(vf, st.pb[qt][f / DT], st.o[qt][f % DT]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Issues a piece's first loads: K of blocks jb, jb+1, jb+2 and V of blocks jb,
// jb+1 into ring stages 0, 1, 2 (stage of block i = (i - jb) % 4).  The piece
// is taken by value: its chunk cursors only move forward, and a pass over the
// piece starts from the caller's unmoved copy.
template <class C>
__device__ __forceinline__ void piece_loads(PieceAddr pa, const AttnArgs& a, uint32_t row_stride,
                                            uint8_t XS_LDS* lds, const uint32_t (&koff)[C::LPW],
                                            const uint32_t (&voff)[C::LPW], int wave) {
  const uint8_t* kbase = (const uint8_t*)a.k + pa.head_off;
  const uint8_t* vbase = (const uint8_t*)a.v + pa.head_off;
  uint8_t XS_LDS* const vlds = lds + C::STAGES * C::TILE;
  load_tile<C>(kbase, row_stride, pa.jb * C::BN, pa.kcur.at(pa.jb), a.S, lds, koff, wave);
  load_tile<C>(vbase, row_stride, pa.jb * C::BN, pa.vcur.at(pa.jb), a.S, vlds, voff, wave);
  if (pa.jb + 1 < pa.je) {
    load_tile<C>(kbase, row_stride, (pa.jb + 1) * C::BN, pa.kcur.at(pa.jb + 1), a.S, lds + C::TILE,
                 koff, wave);
    load_tile<C>(vbase, row_stride, (pa.jb + 1) * C::BN, pa.vcur.at(pa.jb + 1), a.S,
                 vlds + C::TILE, voff, wave);
  }
  if (pa.jb + 2 < pa.je)
    load_tile<C>(kbase, row_stride, (pa.jb + 2) * C::BN, pa.kcur.at(pa.jb + 2), a.S,
                 lds + 2 * C::TILE, koff, wave);
}

// Takes the next piece of the walk and issues its first loads.
template <class C>
__device__ __forceinline__ PieceAddr begin_piece(ShareWalk& walk, const Sched& sch, const AttnArgs& a,
                                                 int nblk, uint32_t row_stride, uint8_t XS_LDS* lds,
                                                 const uint32_t (&koff)[C::LPW],
                                                 const uint32_t (&voff)[C::LPW], int wave, int& slot) {
  PieceAddr pa = next_piece<C::BM, C::ROWB, C::BN>(walk, sch, a, nblk, row_stride, slot);
  piece_loads<C>(pa, a, row_stride, lds, koff, voff, wave);
  return pa;
}

// Loads the piece's query rows (clamped to the sequence) as Q^T B-operand
// fragments, negated when the scale is negative.
template <class C>
__device__ __forceinline__ void load_q(u32x4 (&qf)[C::QT][C::KS], const AttnArgs& a,
                                       const PieceAddr& pa, uint32_t row_stride, uint32_t qflip,
                                       int wave, int lane) {
#pragma unroll
  for (int qt = 0; qt < C::QT; ++qt) {
    int qrow = pa.m0 + wave * C::QW + qt * 32 + (lane & 31);
    qrow = qrow < a.S ? qrow : a.S - 1;
    const long long qr = qrow + (a.chunk_rows ? (long long)(qrow / a.chunk_rows) * a.jump_rows : 0);
    const uint8_t* qp = (const uint8_t*)a.q + pa.head_off + (size_t)qr * row_stride + (lane >> 5) * 16;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qf[qt][ks] = *(const u32x4*)(qp + ks * 32) ^ qflip;
  }
}

// The fast pass's results are usable while every lane's part of every row sum is
// at most 2^40 (false for inf and NaN as well): then no probability exceeded 2^40,
// and O holds at most 2^40 times the largest |v|, far inside the fp32 range.
template <class C>
__device__ __forceinline__ bool sums_ok(const Bf16State<C>& st) {
  bool ok = true;
#pragma unroll
  for (int qt = 0; qt < C::QT; ++qt) ok = ok && st.l[qt] <= 0x1p40f;
  return ok;
}

// One pass over a piece's key blocks jb .. je-1, its first loads already issued.
// CHECK = false (the fast pass): the running max is the piece's first block's
// exact max and stays there, with no overflow checks; the probabilities of later
// blocks may exceed 1 by any factor, which floating point carries without loss
// until the sums leave the range that sums_ok() accepts.  CHECK = true: the lazy
// rescale with the per-block overflow checks above.
template <class C, bool CHECK>
__device__ __forceinline__ void key_pass(Bf16State<C>& st, const AttnArgs& a, PieceAddr pa,
                                         uint32_t row_stride, uint8_t XS_LDS* lds, const LdsOffs<C>& off,
                                         const uint32_t (&koff)[C::LPW], const uint32_t (&voff)[C::LPW],
                                         int wave, int lane, int nfull, float c) {
  constexpr int QT = C::QT, DT = C::DT, BN = C::BN;
  const int S = a.S;
  const int jb = pa.jb, je = pa.je;
  const uint8_t* kbase = (const uint8_t*)a.k + pa.head_off;
  const uint8_t* vbase = (const uint8_t*)a.v + pa.head_off;
  auto kbuf = [&](int s) { return lds + s * C::TILE; };
  auto vbuf = [&](int s) { return lds + (C::STAGES + s) * C::TILE; };
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    st.m[qt] = -INFINITY;
    st.l[qt] = 0.0f;
    st.alpha[qt] = 1.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) st.o[qt][dt] = f32x16{};
  }
  st.rescale = false;

  wait_vmcnt<0>();
  __syncthreads();

  // prologue: score block jb and take its max
  Scores<C> sa, sb;
  qk_block<C>(sa, st, kbuf(0), lane);
  if (jb >= nfull) mask_tail<C>(sa, jb * BN, S, lane);
  softmax_max<C>(st, sa, c);
  if (!CHECK) {
    // O is still zero: no rescale pending; later blocks use this max as is
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) st.alpha[qt] = 1.0f;
    st.rescale = false;
  }

  // K/V blocks stream through a four-stage LDS ring (block i in stage
  // (i - jb) % 4) with one barrier per two blocks: at the barrier before
  // blocks i, i+1 (i - jb even) the loads of K_{i+1}, K_{i+2}, V_i, V_{i+1}
  // (issued at the previous barrier) are complete and every wave is done
  // with blocks i-2, i-1, so K_{i+3}, K_{i+4}, V_{i+2}, V_{i+3} go into the
  // stages those blocks used, one before each of the next four steps (spread
  // out, not all at the barrier where the eight waves' bursts of LDS writes
  // would meet their operand reads: 0.7 % faster).  Entering a step for block
  // i: its scores are in one buffer with their max taken.  Four blocks per
  // trip keep the stages and score buffers static.
  auto ld_k = [&](int i, int stage) {
    load_tile<C>(kbase, row_stride, i * BN, pa.kcur.at(i), S, kbuf(stage), koff, wave);
  };
  auto ld_v = [&](int i, int stage) {
    load_tile<C>(vbase, row_stride, i * BN, pa.vcur.at(i), S, vbuf(stage), voff, wave);
  };
  int j = jb;
  for (; j + 4 < je; j += 4) {
    wait_vmcnt<0>();
    __syncthreads();
    ld_k(j + 3, 3);
    step1<C, 1, CHECK>(sb, sa, st, lds, off, c);  // block j
    if (j + 1 >= nfull) mask_tail<C>(sb, (j + 1) * BN, S, lane);
    ld_v(j + 2, 2);
    step2<C, 0, CHECK>(st, sa, lds, off, c);
    ld_k(j + 4, 0);
    step1<C, 2, CHECK>(sa, sb, st, lds, off, c);  // block j+1
    if (j + 2 >= nfull) mask_tail<C>(sa, (j + 2) * BN, S, lane);
    ld_v(j + 3, 3);
    step2<C, 1, CHECK>(st, sb, lds, off, c);

    wait_vmcnt<0>();
    __syncthreads();
    if (j + 5 < je) ld_k(j + 5, 1);
    step1<C, 3, CHECK>(sb, sa, st, lds, off, c);  // block j+2
    if (j + 3 >= nfull) mask_tail<C>(sb, (j + 3) * BN, S, lane);
    ld_v(j + 4, 0);
    step2<C, 2, CHECK>(st, sa, lds, off, c);
    if (j + 6 < je) ld_k(j + 6, 2);
    step1<C, 0, CHECK>(sa, sb, st, lds, off, c);  // block j+3
    if (j + 4 >= nfull) mask_tail<C>(sa, (j + 4) * BN, S, lane);
    if (j + 5 < je) ld_v(j + 5, 1);
    step2<C, 3, CHECK>(st, sb, lds, off, c);
  }
  // the last one to four blocks j .. je-1 (stages 0..3, scores of block j in sa)
  {
    const int r = je - j;
    wait_vmcnt<0>();
    __syncthreads();
    if (r > 3) ld_k(j + 3, 3);
    if (r > 2) ld_v(j + 2, 2);
    if (r > 3) ld_v(j + 3, 3);
    if (r > 1) {
      step1<C, 1, CHECK>(sb, sa, st, lds, off, c);  // block j
      if (j + 1 >= nfull) mask_tail<C>(sb, (j + 1) * BN, S, lane);
      step2<C, 0, CHECK>(st, sa, lds, off, c);
    }
    if (r > 2) {
      step1<C, 2, CHECK>(sa, sb, st, lds, off, c);  // block j+1
      if (j + 2 >= nfull) mask_tail<C>(sa, (j + 2) * BN, S, lane);
      step2<C, 1, CHECK>(st, sb, lds, off, c);
      wait_vmcnt<0>();
      __syncthreads();
    }
    if (r > 3) {
      step1<C, 3, CHECK>(sb, sa, st, lds, off, c);  // block j+2
      if (j + 3 >= nfull) mask_tail<C>(sb, (j + 3) * BN, S, lane);
      step2<C, 2, CHECK>(st, sa, lds, off, c);
    }
    // the last block, j + r - 1: scores in sa when r is odd (its max not yet
    // taken)
    if (r & 1) {
      if (CHECK) softmax_max<C>(st, sa, c);
      softmax_exp<C>(st, sa, c);
    } else {
      if (CHECK) softmax_max<C>(st, sb, c);
      softmax_exp<C>(st, sb, c);
    }
    pv_only<C, CHECK>(st, lds, off, (uint32_t)(r - 1) * C::TILE);
  }
}

// Persistent workgroups: each walks its share of the schedule (attn_launch.h,
// Sched) piece by piece: whole tiles in rounds, then an equal run of the
// remaining tiles' (tile, key-block pair) units, so no workgroup idles at the
// end and only tiles cut between two shares need a merge.
// Before a piece's output stores, the next piece's first K/V blocks are
// already requested, so the stores drain while those loads are in flight.
template <class C>
__global__ __launch_bounds__(C::THREADS, kGroupsPerCU) void attn_fwd_bf16_kernel(AttnArgs a) {
  constexpr int QT = C::QT, DT = C::DT, BN = C::BN;
  // K stages 0..3 | V stages 0..3
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * C::STAGES * C::TILE];
  __shared__ int vote[C::NW];  // per wave: the fast pass must be redone
  uint8_t XS_LDS* const lds = (uint8_t XS_LDS*)smem;

  const int S = a.S, H = a.H, T = a.T, B = a.B;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const uint32_t row_stride = (uint32_t)H * C::ROWB;  // bytes between consecutive rows
  uint32_t koff[C::LPW], voff[C::LPW];
  tile_offsets<C, false>(row_stride, wave, lane, koff);
  tile_offsets<C, true>(row_stride, wave, lane, voff);
  const int nblk = (S + BN - 1) / BN;
  const int nfull = S / BN;  // blocks with no key past the end of the sequence
  const uint32_t qflip = a.neg ? 0x80008000u : 0u;
  const float c = a.c;
  const LdsOffs<C> off = lds_offsets<C>(lane);

  // this workgroup's share; the workgroups of one XCD take consecutive shares
  const Sched sch{a.units, a.groups, a.npair, a.dp};
  ShareWalk walk;
  walk.init(sch, xcd_tile(blockIdx.x, a.groups));
  if (!walk.more(sch)) return;
  int slot;
  PieceAddr pa = begin_piece<C>(walk, sch, a, nblk, row_stride, lds, koff, voff, wave, slot);
  Bf16State<C> st;
  load_q<C>(st.qf, a, pa, row_stride, qflip, wave, lane);

  for (;;) {
    const int m0 = pa.m0;
    // fast pass; if any wave's row sums left the accepted range, the whole
    // workgroup runs the piece again with the checked lazy rescale
    key_pass<C, false>(st, a, pa, row_stride, lds, off, koff, voff, wave, lane, nfull, c);
    if (lane == 0) vote[wave] = __builtin_amdgcn_ballot_w64(!sums_ok<C>(st)) != 0;
    __syncthreads();
    bool redo = false;
#pragma unroll
    for (int w = 0; w < C::NW; ++w) redo |= vote[w] != 0;
    if (redo) {
      piece_loads<C>(pa, a, row_stride, lds, koff, voff, wave);
      key_pass<C, true>(st, a, pa, row_stride, lds, off, koff, voff, wave, lane, nfull, c);
    }

    // ---- next piece: request its first K/V blocks and its queries before
    // this piece's stores (this piece's Q fragments are no longer needed)
    const bool more = walk.more(sch);
    const PieceAddr cur = pa;
    const int cur_slot = slot;
    if (more) {
      __syncthreads();  // every wave is done reading this piece's tiles
      pa = begin_piece<C>(walk, sch, a, nblk, row_stride, lds, koff, voff, wave, slot);
      load_q<C>(st.qf, a, pa, row_stride, qflip, wave, lane);
    }

    // ---- epilogue
    if (cur.whole) {
      // normalise, round to bf16, store into the destination slice
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const float lrow = sum_halves(st.l[qt]);
        const float inv = a.o_scale / lrow;
        const int srow = m0 + wave * C::QW + qt * 32 + (lane & 31);
        if (a.lse && lane < 32 && srow < S) a.lse[(size_t)cur.bh * S + srow] = row_lse(st.m[qt], lrow);
        if (srow < S) {
          const int p = srow / T;
          const int sp = srow - p * T;
          uint16_t* orow = (uint16_t*)a.out + ((((size_t)p * B + cur.b) * T + sp) * H + cur.h) * C::D;
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
    } else {
      // a tile cut between shares: unnormalised fp32 partials into this
      // share's slot, merged by attn_combine.  O is stored in register order
      // (each 32-row group as D/8 chunks of 64 lanes x 16 bytes), so every
      // store instruction writes 1 KiB contiguously.
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const float lsum = sum_halves(st.l[qt]);
        const int r = wave * C::QW + qt * 32 + (lane & 31);  // row within the tile
        if (m0 + r < S) {
          const size_t sr = (size_t)cur_slot * C::BM + r;
          float* og = a.ws_o + ((size_t)cur_slot * C::BM + wave * C::QW + qt * 32) * C::D;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const f32x16& o = st.o[qt][dt];
              *(f32x4*)(og + ((dt * 4 + r4) * 64 + lane) * 4) =
                  f32x4{o[4 * r4 + 0], o[4 * r4 + 1], o[4 * r4 + 2], o[4 * r4 + 3]};
            }
          if (lane < 32) *(f32x2*)(a.ws_ml + 2 * sr) = f32x2{st.m[qt], lsum};
        }
      }
    }
    if (!more) break;
  }
}

template <class C>
static hipError_t launch_cfg(const AttnArgs& a, hipStream_t stream) {
  if (a.groups < 1) return hipErrorInvalidValue;
  AttnArgs args = a;
  void* kargs[] = {&args};
  return hipLaunchKernel((const void*)attn_fwd_bf16_kernel<C>, dim3((unsigned)a.groups),
                         dim3(C::THREADS), kargs, 0, stream);
}

// Full-height tiles (8 waves), or half-height ones (4 waves, one per SIMD at
// D = 128) for the tiles left over after the whole rounds of a call whose
// schedule cuts no tile: those run as twice as many half tiles instead of
// leaving part of the chip idle for a last, partly filled round.  Half tiles
// are never cut.
template <int D>
static hipError_t launch_d(const AttnArgs& a, hipStream_t stream) {
  using C = Bf16Cfg<D, XS_QT, XS_NW, XS_BN>;
  using CH = Bf16Cfg<D, XS_QT, XS_NW / 2, XS_BN>;
  static_assert(C::BM == kBlockM && CH::BM == kHalfM, "tile geometry");
  if (!a.half) return launch_cfg<C>(a, stream);
  if (a.ws_o != nullptr || a.units != 0) return hipErrorInvalidValue;
  return launch_cfg<CH>(a, stream);
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
