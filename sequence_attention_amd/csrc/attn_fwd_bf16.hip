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
//  * K/V tiles of BN = 64 keys are double buffered in LDS and filled with
//    direct-to-LDS 16-byte buffer loads (no VGPR round trip).  K rows are XOR
//    swizzled for conflict-free ds_read_b128 of the A operand; V rows are
//    swizzled for ds_read_b64_tr_b16, which delivers V^T fragments directly.
//  * Software pipeline inside the wave, one barrier per block:
//      step 1: QK^T of block j+1 (MFMA)  ||  exp/sum/convert of keys 0-31 of block j
//      step 2: P V of block j (MFMA)     ||  exp/sum/convert of keys 32-63 of block j,
//                                            then the row max of block j+1
//    so the matrix core and the vector ALU work on different blocks at once.
//  * Online softmax in base 2: p = 2^(s*c - m), c = scale*log2(e) folded into
//    one FMA per score.  The running max is moved only when a block's max
//    exceeds it by more than 2^TAU (p <= 2^TAU), so rescaling O is a rare
//    wave-uniform branch.  The row sum adds the bf16-rounded p that enter P V.
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
  static constexpr float TAU = 8.0f;     // lazy-rescale threshold (log2 units)
  static_assert(LOADS % NW == 0 && LOADS >= NW, "tile loads must split evenly over waves");
};

#ifndef XS_VSWZ
#define XS_VSWZ 1
#endif

// XOR swizzle of the 16-byte chunk index of V row `row`.  A ds_read_b64_tr_b16
// of a V^T fragment touches 8 rows x 4 chunks and is served one half-wave at a
// time (4 rows x 4 chunks = 256 bytes): XOR-ing the chunk with 4*(row%4) (D=128,
// one row per 256-byte bank line) or 4*((row/2)%2) (D=64, two rows per line)
// puts the 16 chunks of each half-wave on 16 different bank groups.
template <class C>
__device__ __forceinline__ int vswz(int row) {
#if XS_VSWZ == 0
  return (2 * row) & (C::CH - 1);
#else
  constexpr int RPL = 256 / C::ROWB;  // rows per 256-byte bank line
  return 4 * ((row / RPL) & (C::CH / 4 - 1));
#endif
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
  u32x4 pb[C::QT][C::NT][2];  // bf16 probabilities (P^T B-operand fragments)
  float m[C::QT];             // running max of s*c (log2 units), shared by both half-waves
  float l[C::QT];             // lane-local part of the running sum of p
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

// ---- step-2 MFMA work: O^T = alpha O^T + V_j^T P^T
template <class C>
__device__ __forceinline__ void pv_block(Bf16State<C>& st, const uint8_t XS_LDS* sV, int lane) {
  constexpr int QT = C::QT, NT = C::NT, DT = C::DT, CH = C::CH, ROWB = C::ROWB;
  if (st.rescale) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) st.o[qt][dt] *= st.alpha[qt];
      st.alpha[qt] = 1.0f;
    }
    st.rescale = false;
  }
  const int ln = opaque(lane);
  const int g = ln >> 4, L = ln & 15;
  const int vrow = 4 * (g >> 1) + (L >> 2);  // row within an 8-row group
  const int vsw = vswz<C>(vrow);  // rows of a fragment differ from vrow by multiples of 8
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
        for (int qt = 0; qt < QT; ++qt) st.o[qt][dt] = mfma_bf16(vf, st.pb[qt][nt][h], st.o[qt][dt]);
      }
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

// ---- step-2 VALU work: row max of a scored block, lazy move of the running max
template <class C>
__device__ __forceinline__ void softmax_max(Bf16State<C>& st, const Scores<C>& sc, float c) {
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
  }
}

// ---- step-1 VALU work: p = 2^(s c - m) -> bf16 P^T fragments, row sums
template <class C>
__device__ __forceinline__ void keep_probs(const Bf16State<C>& st) {
#pragma unroll
  for (int qt = 0; qt < C::QT; ++qt)
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
      keep(st.pb[qt][nt][0]);
      keep(st.pb[qt][nt][1]);
    }
}

template <class C>
__device__ __forceinline__ void softmax_exp(Bf16State<C>& st, const Scores<C>& sc, float c) {
  constexpr int QT = C::QT, NT = C::NT;
  const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);
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
          lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[i]), ones, lsum, false);
        }
        st.pb[qt][nt][h] = u32x4{w[0], w[1], w[2], w[3]};
      }
    st.l[qt] = lsum;
  }
}

#ifndef XS_LEAD
#define XS_LEAD 3
#endif

// ---- The two steps of the software pipeline, written as fixed sequences of
// micro-steps separated by scheduling barriers: each micro-step reads the LDS
// fragment LEAD positions ahead, issues the MFMA that uses the fragment read
// LEAD micro-steps earlier, and does a slice of the softmax work, so LDS
// latency and vector work hide under the matrix core.  The exponentials of a
// block are split between the two steps (keys 0-31 under the next block's
// QK^T, keys 32-63 under the first half of this block's P V) so that neither
// step is bound by the vector ALU.  LDS addresses are per-lane offsets
// computed once plus immediates (the double-buffer stage is a template
// argument: splits start on even blocks).

// Per-lane LDS byte offsets of the fragments, relative to a tile's start.
template <class C>
struct LdsOffs {
  uint32_t k[C::KS];  // K fragment of k-step ks (row lane%32, chunk 2ks + lane/32)
  uint32_t v[C::DT];  // first V^T transpose read of d-tile dt (rows 0..7 group)
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
    o.v[dt] = (uint32_t)(vrow * C::ROWB + 8 * (L & 1) + (chunk << 4));
  }
  return o;
}

// exp2(s c - m) of score pair e (0..7) of 32-key tile nt, query sub-tile qt,
// packed to bf16, added to the row sum; pinned to the current micro-step.
template <class C>
__device__ __forceinline__ void exp_pair(const Scores<C>& cur, int qt, int nt, int e, float c,
                                         float neg_m, float& lsum, uint32_t& w) {
  const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);
  const float p0 = fast_exp2(__builtin_fmaf(cur.s[nt][qt][2 * e], c, neg_m));
  const float p1 = fast_exp2(__builtin_fmaf(cur.s[nt][qt][2 * e + 1], c, neg_m));
  uint32_t pk = pack_bf16(p0, p1);
  lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), ones, lsum, false);
  pin(pk);
  pin(lsum);
  w = pk;
}

// Step 1: S^T of the next block from K stage KST || probabilities of keys 0..31
// of the current block.  Each K fragment feeds the QT query sub-tiles.
template <class C, int KST>
__device__ __forceinline__ void step1(Scores<C>& nxt, const Scores<C>& cur, Bf16State<C>& st,
                                      const uint8_t XS_LDS* lds, const LdsOffs<C>& off, float c) {
  static_assert(C::NT == 2, "pipeline written for 64-key blocks");
  constexpr int QT = C::QT, NT = C::NT, KS = C::KS, ROWB = C::ROWB;
  constexpr int NF = KS * NT;
  constexpr int LEAD = XS_LEAD < NF ? XS_LEAD : NF;
  constexpr int R = LEAD + 1;
  constexpr int NE = 8 * QT;  // score pairs of keys 0..31, all sub-tiles
  const uint8_t XS_LDS* kb = lds + KST * C::TILE;
  auto kread = [&](int f) { return lds_read_b128(kb + off.k[f / NT] + (f % NT) * 32 * ROWB); };
  float neg_m[QT], lsum[QT];
  uint32_t w[QT][8];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    neg_m[qt] = -st.m[qt];
    lsum[qt] = st.l[qt];
  }
  u32x4 kf[R];
#pragma unroll
  for (int f = 0; f < LEAD; ++f) kf[f] = kread(f);
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    if (f + LEAD < NF) kf[(f + LEAD) % R] = kread(f + LEAD);
    const int ks = f / NT, nt = f % NT;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
      nxt.s[nt][qt] = mfma_bf16(kf[f % R], st.qf[qt][ks], ks == 0 ? f32x16{} : nxt.s[nt][qt]);
    // the score pairs of tile 0, spread evenly over the NF micro-steps
#pragma unroll
    for (int e = 0; e < NE; ++e)
      if (e * NF / NE == f) exp_pair<C>(cur, e / 8, 0, e % 8, c, neg_m[e / 8], lsum[e / 8], w[e / 8][e % 8]);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    st.l[qt] = lsum[qt];
    st.pb[qt][0][0] = u32x4{w[qt][0], w[qt][1], w[qt][2], w[qt][3]};
    st.pb[qt][0][1] = u32x4{w[qt][4], w[qt][5], w[qt][6], w[qt][7]};
    keep(st.pb[qt][0][0]);
    keep(st.pb[qt][0][1]);
  }
}

// Step 2: O^T = alpha O^T + V^T P^T from V stage VST; under the first half
// (keys 0..31) the probabilities of keys 32..63, under the second half the row
// max of the next block (lazy move of the running max; the O rescale it may
// ask for is applied at the start of the next step 2).
template <class C, int VST>
__device__ __forceinline__ void step2(Bf16State<C>& st, const Scores<C>& nxt, const Scores<C>& cur,
                                      const uint8_t XS_LDS* lds, const LdsOffs<C>& off, float c) {
  constexpr int QT = C::QT, NT = C::NT, DT = C::DT, ROWB = C::ROWB;
  constexpr int NF = NT * 2 * DT;          // V fragments, keys 0..31 first
  constexpr int HALF = NF / 2;
  constexpr int LEAD = XS_LEAD < NF ? XS_LEAD : NF;
  constexpr int R = LEAD + 1;
  constexpr int NE = 8 * QT;               // score pairs of keys 32..63
  constexpr int NM = 32 * QT;              // scores of the next block per lane
  if (st.rescale) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) st.o[qt][dt] *= st.alpha[qt];
      st.alpha[qt] = 1.0f;
    }
    st.rescale = false;
  }
  const uint8_t XS_LDS* vb = lds + (2 + VST) * C::TILE;
  auto vaddr = [&](int f) {
    const int nt = f / (2 * DT), h = (f / DT) % 2, dt = f % DT;
    return vb + off.v[dt] + (nt * 32 + 16 * h) * ROWB;
  };
  float neg_m[QT], lsum[QT], mx[QT];
  uint32_t w[QT][8];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    neg_m[qt] = -st.m[qt];
    lsum[qt] = st.l[qt];
    mx[qt] = nxt.s[0][qt][0];
  }
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
    if (f == HALF) {
      // probabilities of keys 32..63 complete: assemble their operands
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        st.pb[qt][1][0] = u32x4{w[qt][0], w[qt][1], w[qt][2], w[qt][3]};
        st.pb[qt][1][1] = u32x4{w[qt][4], w[qt][5], w[qt][6], w[qt][7]};
      }
    }
    const int nt = f / (2 * DT), h = (f / DT) % 2, dt = f % DT;
    const u32x4 vf = u32x4{vlo[f % R][0], vlo[f % R][1], vhi[f % R][0], vhi[f % R][1]};
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) st.o[qt][dt] = mfma_bf16(vf, st.pb[qt][nt][h], st.o[qt][dt]);
    if (f < HALF) {
#pragma unroll
      for (int e = 0; e < NE; ++e)
        if (e * HALF / NE == f)
          exp_pair<C>(cur, e / 8, 1, e % 8, c, neg_m[e / 8], lsum[e / 8], w[e / 8][e % 8]);
    } else {
      constexpr int EPS = NM / HALF;  // max over the scores of the next block
#pragma unroll
      for (int ee = 0; ee < EPS; ++ee) {
        const int e = (f - HALF) * EPS + ee;  // 0 .. NM-1
        const int qt = e / 32, r = e % 32;
        mx[qt] = fmaxf(mx[qt], nxt.s[r / 16][qt][r % 16]);
      }
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) pin(mx[qt]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  bool need[QT], any = false;
  float mnew[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    st.l[qt] = lsum[qt];
    mnew[qt] = max_halves(mx[qt]) * c;
    need[qt] = mnew[qt] > st.m[qt] + C::TAU;
    any |= need[qt];
  }
  if (__builtin_amdgcn_ballot_w64(any)) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float a = need[qt] ? fast_exp2(st.m[qt] - mnew[qt]) : 1.0f;
      st.m[qt] = need[qt] ? mnew[qt] : st.m[qt];
      st.l[qt] *= a;
      st.alpha[qt] *= a;
    }
    st.rescale = true;
  }
}

// Takes the next piece of the walk and issues its first loads (K and V of
// block jb into stage 0, K of jb+1 into stage 1).
template <class C>
__device__ __forceinline__ PieceAddr begin_piece(ShareWalk& walk, const Sched& sch, const AttnArgs& a,
                                                 int nblk, uint32_t row_stride, uint8_t XS_LDS* lds,
                                                 const uint32_t (&koff)[C::LPW],
                                                 const uint32_t (&voff)[C::LPW], int wave, int& slot) {
  PieceAddr pa = next_piece<C::BM, C::ROWB>(walk, sch, a, nblk, row_stride, slot);
  const uint8_t* kbase = (const uint8_t*)a.k + pa.head_off;
  const uint8_t* vbase = (const uint8_t*)a.v + pa.head_off;
  load_tile<C>(kbase, row_stride, pa.jb * C::BN, pa.kcur.at(pa.jb), a.S, lds, koff, wave);
  load_tile<C>(vbase, row_stride, pa.jb * C::BN, pa.vcur.at(pa.jb), a.S, lds + 2 * C::TILE, voff,
               wave);
  if (pa.jb + 1 < pa.je)
    load_tile<C>(kbase, row_stride, (pa.jb + 1) * C::BN, pa.kcur.at(pa.jb + 1), a.S, lds + C::TILE,
                 koff, wave);
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

// Persistent workgroups: each walks its share of the schedule (attn_launch.h,
// Sched) piece by piece: whole tiles in rounds, then an equal run of the
// remaining tiles' (tile, key-block pair) units, so no workgroup idles at the
// end and only tiles cut between two shares need a merge.
// Before a piece's output stores, the next piece's first K/V blocks are
// already requested, so the stores drain while those loads are in flight.
template <class C>
__global__ __launch_bounds__(C::THREADS, kGroupsPerCU) void attn_fwd_bf16_kernel(AttnArgs a) {
  constexpr int QT = C::QT, DT = C::DT, BN = C::BN;
  // K stage 0 | K stage 1 | V stage 0 | V stage 1
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * C::TILE];
  uint8_t XS_LDS* const lds = (uint8_t XS_LDS*)smem;
  auto kbuf = [&](int i) { return lds + (i & 1) * C::TILE; };
  auto vbuf = [&](int i) { return lds + (2 + (i & 1)) * C::TILE; };

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
    const int jb = pa.jb, je = pa.je, m0 = pa.m0;
    const uint8_t* kbase = (const uint8_t*)a.k + pa.head_off;
    const uint8_t* vbase = (const uint8_t*)a.v + pa.head_off;

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
    qk_block<C>(sa, st, kbuf(jb), lane);
    if (jb >= nfull) mask_tail<C>(sa, jb * BN, S, lane);
    softmax_max<C>(st, sa, c);

    // Steady state, two blocks per trip so the score buffers swap statically.
    // Entering a step for block i: scores of block i are in one buffer with
    // their max taken; K_{i+1} and V_i are loaded (or in flight).
    // (jb is even: K_i and V_i live in stage i % 2)
    int j = jb;
    for (; j + 2 < je; j += 2) {
      // ---- block j (scores in sa), next block's scores into sb
      wait_vmcnt<0>();
      __syncthreads();
      load_tile<C>(kbase, row_stride, (j + 2) * BN, pa.kcur.at(j + 2), S, kbuf(0), koff, wave);
      load_tile<C>(vbase, row_stride, (j + 1) * BN, pa.vcur.at(j + 1), S, vbuf(1), voff, wave);
      step1<C, 1>(sb, sa, st, lds, off, c);
      if (j + 1 >= nfull) mask_tail<C>(sb, (j + 1) * BN, S, lane);
      step2<C, 0>(st, sb, sa, lds, off, c);

      // ---- block j+1 (scores in sb), next block's scores into sa
      wait_vmcnt<0>();
      __syncthreads();
      if (j + 3 < je)
        load_tile<C>(kbase, row_stride, (j + 3) * BN, pa.kcur.at(j + 3), S, kbuf(1), koff, wave);
      load_tile<C>(vbase, row_stride, (j + 2) * BN, pa.vcur.at(j + 2), S, vbuf(0), voff, wave);
      step1<C, 0>(sa, sb, st, lds, off, c);
      if (j + 2 >= nfull) mask_tail<C>(sa, (j + 2) * BN, S, lane);
      step2<C, 1>(st, sa, sb, lds, off, c);
    }
    // the last one or two blocks (scores of block j in sa)
    if (j + 1 < je) {
      wait_vmcnt<0>();
      __syncthreads();
      load_tile<C>(vbase, row_stride, (j + 1) * BN, pa.vcur.at(j + 1), S, vbuf(j + 1), voff, wave);
      qk_block<C>(sb, st, kbuf(j + 1), lane);
      softmax_exp<C>(st, sa, c);
      __builtin_amdgcn_sched_barrier(0);
      if (j + 1 >= nfull) mask_tail<C>(sb, (j + 1) * BN, S, lane);
      pv_block<C>(st, vbuf(j), lane);
      softmax_max<C>(st, sb, c);
      wait_vmcnt<0>();
      __syncthreads();
      softmax_exp<C>(st, sb, c);
      pv_block<C>(st, vbuf(j + 1), lane);
    } else {
      wait_vmcnt<0>();  // V_j may have been issued by the last loop step
      __syncthreads();
      softmax_exp<C>(st, sa, c);
      pv_block<C>(st, vbuf(j), lane);
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
      // share's slot, merged by attn_combine
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const float lsum = sum_halves(st.l[qt]);
        const int r = wave * C::QW + qt * 32 + (lane & 31);  // row within the tile
        if (m0 + r < S) {
          const size_t sr = (size_t)cur_slot * C::BM + r;
          float* orow = a.ws_o + sr * C::D;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const f32x16& o = st.o[qt][dt];
              *(f32x4*)(orow + dt * 32 + r4 * 8 + 4 * (lane >> 5)) =
                  f32x4{o[4 * r4 + 0], o[4 * r4 + 1], o[4 * r4 + 2], o[4 * r4 + 3]};
            }
          if (lane < 32) *(f32x2*)(a.ws_ml + 2 * sr) = f32x2{st.m[qt], lsum};
        }
      }
    }
    if (!more) break;
  }
}

template <int D>
static hipError_t launch_d(const AttnArgs& a, hipStream_t stream) {
  using C = Bf16Cfg<D, XS_QT, XS_NW, XS_BN>;
  static_assert(C::BM == kBlockM && C::BN == kBlockN, "tile geometry");
  if (a.groups < 1) return hipErrorInvalidValue;
  AttnArgs args = a;
  void* kargs[] = {&args};
  return hipLaunchKernel((const void*)attn_fwd_bf16_kernel<C>, dim3((unsigned)a.groups),
                         dim3(C::THREADS), kargs, 0, stream);
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
