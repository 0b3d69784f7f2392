// attn_fwd_fp8.hip -- the attention forward pass over OCP e4m3 (e4m3fn) Q/K/V
// with per-tensor descales, fp32 accumulation and bf16 output, fused with the
// destination-ordered epilogue; gfx950.
//
// Same operation as the bf16 kernel (X-Stage paper, catalyzex.com abstract;
// gist.science explainer, "Zentrale Beitraege", "FlashAttention-A2A
// (Piggybacking)"): per workgroup 8 waves x 32 query rows of one (b, h), K/V
// blocks of 64 keys in a four-stage LDS ring filled by direct-to-LDS loads
// (one barrier per two blocks), a software pipeline of pinned micro-steps
// inside each wave.  What differs for 8-bit operands:
//  * Both contractions use v_mfma_f32_32x32x64_f8f6f4 (e4m3 x e4m3 -> fp32):
//    S^T = K Q^T takes D/64 k-steps; O^T += V^T P^T takes one k-step of all 64
//    keys of the block per 32-row d tile.
//  * The descales fold into the exponent factor (c = scale*dq*dk*log2 e) and
//    the epilogue (O * dv / l); the MFMAs see the raw e4m3 codes.
//  * P enters P V as e4m3.  With the log-sum-exp output it is p = 2^(s c - m)
//    rounded to e4m3 (p <= 2^TAU = 256 < 448, so nothing saturates); without
//    it, the e4m3 code of each probability is read off its exponent by one FMA
//    and one integer conversion, with no exponential (code4).
//    The accumulator registers of the scores already hold, per half-wave, the
//    32 keys
//    {8g + 4h + i}; the V tile is stored in LDS with its rows permuted so that
//    those keys are 32 consecutive rows, which ds_read_b64_tr_b8 turns into
//    the V^T operand in the same order.
//  * The row sums that normalise O are those of the quantised P, computed on
//    the matrix core: one more (16x16x128) MFMA per block with a selector A
//    operand (the vector ALU, not the matrix core, bounds this kernel).  When the
//    log-sum-exp output is requested, a second instantiation instead adds the
//    fp32 probabilities before quantisation and normalises with that sum,
//    which the log-sum-exp is defined by.  Having those sums at hand, it also
//    skips the per-block row max: a lane whose sum of a block's new
//    probabilities exceeds 2^TAU (as any single one above 2^TAU makes it)
//    triggers the block's exact max, the lazy move and a recomputation, before
//    P V uses the block.
#include "attn_launch.h"
#include "device_common.h"
#include "piece.h"

namespace xs {

template <int D_, bool LSE_, int NW_ = 8>
struct Fp8Cfg {
  static constexpr int D = D_;
  static constexpr bool LSE = LSE_;       // also keep fp32 row sums for the log-sum-exp output
  static constexpr int NW = NW_;          // waves per workgroup, 32 query rows each
  static constexpr int BN = 64;           // keys per K/V block
  static constexpr int QW = 32;
  static constexpr int BM = QW * NW;
  static constexpr int ROWB = D;          // bytes per K/V row
  static constexpr int CH = D / 16;       // 16-byte chunks per row
  static constexpr int RPB = 256 / D;     // rows per 256 bytes (one pass over the LDS banks)
  static constexpr int TILE = BN * ROWB;  // bytes per K or V tile
  static constexpr int LOADS = TILE / 1024;
  static constexpr int KS = D / 64;       // k-steps of QK^T
  static constexpr int DT = D / 32;       // 32-row d tiles of O^T
  static constexpr int NT = BN / 32;      // 32-key score tiles per block
  static constexpr int THREADS = 64 * NW;
  static constexpr int STAGES = 4;        // LDS ring depth for K and for V
  // lazy-rescale threshold (log2 units): every x = s c - m stays <= TAU
  static constexpr float TAU = LSE_ ? 8.0f : 4.0f;
  static constexpr float PMAX = LSE_ ? 256.0f : 16.0f;  // 2^TAU
  // Without the log-sum-exp: P = 2^(x + SHIFT) as e4m3 codes (code4); the codes
  // of x in [-6 - SHIFT, TAU] are normal e4m3 numbers and the largest, x = TAU,
  // is code 126 (448), one below the NaN code.
  static constexpr float SHIFT = 4.75f;
  static constexpr float CODE_BIAS = 8.0f * (SHIFT + 7.0f);
  // 1 KiB direct loads per wave and tile: one (the first LOADS waves), or
  // LOADS / NW when there are fewer waves than loads
  static constexpr int LPW = LOADS > NW ? LOADS / NW : 1;
  static_assert(LOADS <= NW || LOADS % NW == 0, "tile loads must split evenly over waves");
  static_assert(NT == 2, "the P^T operand layout assumes 64-key blocks");
};

// LDS row R of a V tile holds key 8*((R%32)/4) + 4*(R/32) + R%4: rows
// 32h..32h+31 are the keys whose scores half-wave h holds, in register order.
__device__ __forceinline__ int vrow_key(int R) { return 8 * ((R & 31) >> 2) + 4 * (R >> 5) + (R & 3); }

// XOR swizzles of the 16-byte chunk index, chosen so that a ds_read_b128 of
// 16 consecutive K rows, and a ds_read_b64_tr_b8 of 8 V rows x 2 chunks, touch
// every LDS bank once.
template <class C>
__device__ __forceinline__ int kswz(int R) { return (R / C::RPB) & (C::CH - 1); }
template <class C>
__device__ __forceinline__ int vswz(int R) { return 2 * ((R / C::RPB) & (C::CH / 2 - 1)); }

template <class C>
__device__ __forceinline__ void load_tile8(const uint8_t* head_base, uint32_t row_stride, int kv0,
                                           size_t extra, int S, const uint8_t XS_LDS* dst,
                                           const uint32_t (&voff)[C::LPW], int wave) {
  if constexpr (C::LPW == 1) {
    if (wave < C::LOADS) {
      const u32x4 rsrc = make_rsrc(head_base + (size_t)kv0 * row_stride + extra,
                                   (uint32_t)(S - kv0 - 1) * row_stride + (uint32_t)C::ROWB);
      load_lds_b128(rsrc, voff[0], lds_addr(dst) + (uint32_t)wave * 1024u);
    }
  } else {
    const u32x4 rsrc = make_rsrc(head_base + (size_t)kv0 * row_stride + extra,
                                 (uint32_t)(S - kv0 - 1) * row_stride + (uint32_t)C::ROWB);
#pragma unroll
    for (int i = 0; i < C::LPW; ++i)
      load_lds_b128(rsrc, voff[i], lds_addr(dst) + (uint32_t)(wave * C::LPW + i) * 1024u);
  }
}

template <class C>
struct Scores8 {
  f32x16 s[C::NT];
};

template <class C>
struct Fp8State {
  f32x16 o[C::DT];
  f32x4 lt;          // row sums of the quantised P: lane n < 16 holds query n's in register 0 and
                     // query n+16's in register 1 (16x16 layout of the row-sum MFMA)
  i32x8 qf[C::KS];
  u32x4 p0, p1;      // P^T operand: e4m3 probabilities of keys 0..31 and 32..63
  float m, alpha;
  float l32;         // lane-local fp32 sum of the unquantised p (kept only when C::LSE)
  float lb;          // l32 before the current block's probabilities (C::LSE)
  float mx0;         // lane max of the next block's key tile 0 (end of step A, without C::LSE)
  bool rescale;
};

// The A operand of the row-sum MFMA, lt += SEL P^T with the 16x16x128 e4m3
// instruction (half the matrix-core time of a 32x32x64 one): each query's sum
// of the quantised probabilities of the block, accumulated in lane n < 16,
// register 0 (query n) and register 1 (query n+16).
__device__ __forceinline__ i32x8 ones_e4m3(int lane) {
  // A operand of v_mfma_f32_16x16x128_f8f6f4, lane l = row l%16, k = 32(l/16) ..
  // 32(l/16)+31.  The P^T operand, read as that instruction's B operand, gives
  // column n the bytes of lanes n, n+16, n+32, n+48: query n's keys 0..31, query
  // n+16's keys 0..31, query n's keys 32..63, query n+16's keys 32..63.  Row 0
  // (e4m3 1.0 on k groups 0 and 2) sums query n's, row 1 (groups 1 and 3) query
  // n+16's; the other rows are zero.
  const int row = lane & 15, g = lane >> 4;
  const int w = (row == 0 && (g & 1) == 0) || (row == 1 && (g & 1) == 1) ? 0x38383838 : 0;
  return i32x8{w, w, w, w, w, w, w, w};
}
__device__ __forceinline__ f32x4 mfma_rowsum(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <class C>
__device__ __forceinline__ void qk_block8(Scores8<C>& sc, const Fp8State<C>& st,
                                          const uint8_t XS_LDS* sK, int lane) {
  const int ln = opaque(lane);
  const int hi = ln >> 5;
  const int R = ln & 31;
  const uint8_t XS_LDS* krow = sK + R * C::ROWB;
  const int sw = kswz<C>(R);
#pragma unroll
  for (int t = 0; t < C::KS; ++t) {
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
      const int c0 = 4 * t + 2 * hi;
      const u32x4 a0 = lds_read_b128(krow + nt * 32 * C::ROWB + ((c0 ^ sw) << 4));
      const u32x4 a1 = lds_read_b128(krow + nt * 32 * C::ROWB + (((c0 + 1) ^ sw) << 4));
      const i32x8 kf = __builtin_bit_cast(i32x8, (u32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]}));
      sc.s[nt] = mfma_fp8(kf, st.qf[t], t == 0 ? f32x16{} : sc.s[nt]);
    }
  }
}

template <class C>
__device__ __forceinline__ void mask_tail8(Scores8<C>& sc, int kv0, int S, int lane) {
  const int hi = lane >> 5;
#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kv0 + nt * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
      if (key >= S) sc.s[nt][r] = -INFINITY;
    }
}

// Masks a partial block that step A has just scored.  Without the log-sum-exp,
// step A already took the lane max of its key tile 0 for step B: take it again
// without the masked keys.
template <class C>
__device__ __forceinline__ void mask_tail_next8(Scores8<C>& sc, Fp8State<C>& st, int kv0, int S, int lane) {
  mask_tail8<C>(sc, kv0, S, lane);
  if (!C::LSE) {
    float mx = sc.s[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc.s[0][r]);
    st.mx0 = mx;
  }
}

template <class C>
__device__ __forceinline__ bool softmax_max8(Fp8State<C>& st, const Scores8<C>& sc, float c) {
  float mx = sc.s[0][0];
#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc.s[nt][r]);
  const float mnew = max_halves(mx) * c;
  const bool need = mnew > st.m + C::TAU;
  if (__builtin_amdgcn_ballot_w64(need)) {
    const float a = need ? fast_exp2(st.m - mnew) : 1.0f;
    st.m = need ? mnew : st.m;
    st.alpha *= a;
    if (C::LSE) st.l32 *= a;
    st.rescale = true;
    return true;
  }
  return false;
}

// The row sum that normalises O: without the log-sum-exp output, the sum of
// the quantised probabilities that entered P V (from the row-sum MFMA; every
// register of lt holds it); with it, the fp32 sum of the unquantised
// probabilities (the sum the log-sum-exp is defined by).
template <class C>
__device__ __forceinline__ float row_sum(const Fp8State<C>& st) {
  if (C::LSE) return sum_halves(st.l32);
  const int lane = __lane_id(), src = (lane & 15) << 2;
  const float r0 = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(st.lt[0])));
  const float r1 = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(st.lt[1])));
  return (lane & 16) ? r1 : r0;
}

// O^T and the row sums *= alpha (rare: only when the running max moved).
template <class C>
__device__ __forceinline__ void rescale_o8(Fp8State<C>& st) {
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) {
    st.o[dt] *= st.alpha;
    __builtin_amdgcn_sched_barrier(0);
  }
  if (!C::LSE) {
    // lane n < 16: register 0 is query n's (alpha of this lane), register 1 query n+16's
    const int src = ((__lane_id() + 16) & 63) << 2;
    st.lt[0] *= st.alpha;
    st.lt[1] *= __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(st.alpha)));
  }
  st.alpha = 1.0f;
  st.rescale = false;
}

#ifndef XS_LEAD8
#define XS_LEAD8 1
#endif

// ---- The software pipeline as fixed sequences of micro-steps (one MFMA each,
// separated by scheduling barriers, the vector work of each micro-step pinned
// in place).  One PV MFMA of the fp8 kernel takes all 64 keys of a block, so
// the probabilities of a block must be complete before its first PV MFMA; the
// work is therefore split as
//   step A: QK^T of block j+1 (MFMA)  ||  probabilities of keys 32..63 of block j
//   step B: P V of block j (MFMA)     ||  row max of block j+1, lazy move of the
//                                         running max, probabilities of its keys 0..31
// so that each step carries about half of the vector work.

// Per-lane LDS byte offsets of the fragments, relative to a tile's start.
template <class C>
struct LdsOffs8 {
  uint32_t k[C::KS][2];  // the two 16-byte K chunks of k-step ks (row lane%32)
  uint32_t v[C::DT];     // first transpose read of d-tile dt (then + 8 rows each)
};

template <class C>
__device__ __forceinline__ LdsOffs8<C> lds_offsets8(int lane) {
  LdsOffs8<C> o;
  const int hi = lane >> 5, R = lane & 31, sw = kswz<C>(R);
#pragma unroll
  for (int t = 0; t < C::KS; ++t) {
    const int c0 = 4 * t + 2 * hi;
    o.k[t][0] = (uint32_t)(R * C::ROWB + ((c0 ^ sw) << 4));
    o.k[t][1] = (uint32_t)(R * C::ROWB + (((c0 + 1) ^ sw) << 4));
  }
  const int g = lane >> 4, L = lane & 15, h = g >> 1;
  const int R0 = 32 * h + (L >> 1);
  const int vs = vswz<C>(R0);  // the same for R0 + 8t
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) {
    const int chunk = (dt * 2 + (g & 1)) ^ vs;
    o.v[dt] = (uint32_t)(R0 * C::ROWB + 8 * (L & 1) + (chunk << 4));
  }
  return o;
}

// Four fp32 values -> four OCP e4m3 bytes (round to nearest even), first value
// in the low byte.  Inputs must stay below 464 (larger values become NaN).  The
// first conversion writes the low half and keeps the high half of its `old`
// operand, which the second conversion overwrites: any register will do as
// `old`, so a's own bits are passed and no zeroed register is needed.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// The probabilities of scores 4q..4q+3 of 32-key tile nt in two halves, a
// micro-step apart, so the conversion never waits on the transcendental
// unit's latency: exp4 computes p = 2^(s c - m), pack4 rounds them to four
// e4m3 bytes.  Both are pinned to the micro-step they are issued in.
template <class C>
__device__ __forceinline__ f32x4 exp4(const Scores8<C>& sc, int nt, int q, float c, float neg_m,
                                      float& lsum) {
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p[i] = fast_exp2(__builtin_fmaf(sc.s[nt][4 * q + i], c, neg_m));
    if (C::LSE) lsum += p[i];
    pin(p[i]);
  }
  if (C::LSE) pin(lsum);
  return f32x4{p[0], p[1], p[2], p[3]};
}

__device__ __forceinline__ uint32_t pack4(f32x4 p) {
  uint32_t pk = pack_e4m3x4(p[0], p[1], p[2], p[3]);
  pin(pk);
  return pk;
}

// Without the log-sum-exp output the probabilities are not exponentiated: an
// e4m3 number is 2^(E - 7) (1 + M/8) with code 8E + M, so for y = x + SHIFT
// = e + f (e integer, f in [0, 1)) the code round(8 (y + 7)) encodes 2^e (1 + f)
// -- 2^y interpolated linearly between powers of two (within +6.2 % of it), on
// e4m3's three-bit mantissa grid (within half a step, 6.25 %).  One FMA gives
// z = 8 (y + 7) / 65535 = s (8c / 65535) + 8 (SHIFT + 7 - m) / 65535, and a
// normalised 16-bit conversion (v_cvt_pknorm_u16_f32: clamp to [0, 1], times
// 65535, rounded to the nearest integer) turns two such values into two codes at
// once; one byte permutation packs four.  The row sums that normalise O are those
// of the same codes' values (row-sum MFMA), and the constant 2^SHIFT cancels in
// O / l.  x <= TAU = 4 keeps every code <= 126 (so the low byte of each 16-bit
// result is the code); x < -10.75 gives subnormal codes and x below about -11.7
// code 0: weights under 2^-10.75 of the row's largest key (which has x >= 0).
// code4 computes the four values z as fp32 (pinned), pack_codes4 packs the codes.
template <class C>
__device__ __forceinline__ f32x4 code4(const Scores8<C>& sc, int nt, int q, float c8, float bias) {
  float t[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    t[i] = __builtin_fmaf(sc.s[nt][4 * q + i], c8, bias);
    pin(t[i]);
  }
  return f32x4{t[0], t[1], t[2], t[3]};
}
__device__ __forceinline__ uint32_t pack_codes4(f32x4 t) {
  // codes 0 and 1 in the low bytes of lo's halves, codes 2 and 3 in hi's;
  // selector bytes 0, 2 pick lo's bytes 0, 2 and 4, 6 hi's bytes 0, 2
  const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pknorm_u16(t[0], t[1]));
  const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pknorm_u16(t[2], t[3]));
  uint32_t w = __builtin_amdgcn_perm(hi, lo, 0x06040200u);
  pin(w);
  return w;
}
// The instantiation's form of the probabilities: exp4/pack4 with the
// log-sum-exp (factors (a, b) = (c, -m)), code4/pack_codes4 without it
// ((a, b) = (8c, 8(-m) + CODE_BIAS) / 65535).
template <class C>
__device__ __forceinline__ float prob_a(float c) { return C::LSE ? c : 8.0f * c * (1.0f / 65535.0f); }
template <class C>
__device__ __forceinline__ float prob_b(float neg_m) {
  return C::LSE ? neg_m : (8.0f * neg_m + C::CODE_BIAS) * (1.0f / 65535.0f);
}
template <class C>
__device__ __forceinline__ f32x4 prob4(const Scores8<C>& sc, int nt, int q, float a, float b,
                                       float& lsum) {
  if (C::LSE) return exp4<C>(sc, nt, q, a, b, lsum);
  return code4<C>(sc, nt, q, a, b);
}
template <class C>
__device__ __forceinline__ uint32_t packp4(f32x4 p) {
  return C::LSE ? pack4(p) : pack_codes4(p);
}

// Probabilities of all 32 keys of tile nt (prologue and tail, not pipelined).
template <class C>
__device__ __forceinline__ void exp_tile8(Fp8State<C>& st, const Scores8<C>& sc, int nt, float c,
                                          u32x4& out) {
  const float neg_m = -st.m;
  float lsum = st.l32;
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    w[q] = packp4<C>(prob4<C>(sc, nt, q, prob_a<C>(c), prob_b<C>(neg_m), lsum));
  st.l32 = lsum;
  out = u32x4{w[0], w[1], w[2], w[3]};
}

// Step A: S^T of the next block from K stage KST || keys 32..63 of the current
// block (its keys 0..31 were done in the previous step B).
template <class C, int KST>
__device__ __forceinline__ void step_a8(Scores8<C>& nxt, const Scores8<C>& cur, Fp8State<C>& st,
                                        const uint8_t XS_LDS* lds, const LdsOffs8<C>& off, float c) {
  constexpr int NT = C::NT, KS = C::KS, ROWB = C::ROWB;
  constexpr int NF = KS * NT;
  constexpr int LEAD = XS_LEAD8 < NF ? XS_LEAD8 : NF;
  constexpr int R = LEAD + 1;
  const uint8_t XS_LDS* kb = lds + KST * C::TILE;
  auto kread = [&](int f) {
    const int t = f / NT, nt = f % NT;
    const u32x4 a0 = lds_read_b128(kb + off.k[t][0] + nt * 32 * ROWB);
    const u32x4 a1 = lds_read_b128(kb + off.k[t][1] + nt * 32 * ROWB);
    return __builtin_bit_cast(i32x8, (u32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]}));
  };
  const float neg_m = -st.m;
  const float pa = prob_a<C>(c), pb = prob_b<C>(neg_m);
  float lsum = st.l32;
  uint32_t w[4];
  f32x4 pe[4];
  i32x8 kf[R];
#pragma unroll
  for (int f = 0; f < LEAD; ++f) kf[f] = kread(f);
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    if (f + LEAD < NF) kf[(f + LEAD) % R] = kread(f + LEAD);
    const int t = f / NT, nt = f % NT;
    nxt.s[nt] = mfma_fp8(kf[f % R], st.qf[t], t == 0 ? f32x16{} : nxt.s[nt]);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (f > 0 && q * NF / 4 == f - 1) w[q] = packp4<C>(pe[q]);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (q * NF / 4 == f) pe[q] = prob4<C>(cur, 1, q, pa, pb, lsum);
    if (!C::LSE && f == NF - 1) {
      // the next block's key tile 0 is complete (its last k-step was the MFMA
      // before this one): half of its row max here, the other half in step B
      float mx = nxt.s[0][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, nxt.s[0][r]);
      pin(mx);
      st.mx0 = mx;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (q * NF / 4 == NF - 1) w[q] = packp4<C>(pe[q]);
  st.l32 = lsum;
  st.p1 = u32x4{w[0], w[1], w[2], w[3]};
  keep(st.p1);
  if (C::LSE) {
    // Overflow check of the block's probabilities (keys 0..31 from the step B
    // before, 32..63 here; none has entered P V yet): a lane whose sum of them
    // exceeds 2^TAU may hold one above 2^TAU.  Then the block's exact max is
    // taken and, if the running max moves, all 64 are recomputed with it (the
    // O rescale waits for step B).
    if (__builtin_amdgcn_ballot_w64(!(st.l32 - st.lb <= C::PMAX))) {
      st.l32 = st.lb;
      if (softmax_max8<C>(st, cur, c)) {
        exp_tile8<C>(st, cur, 0, c, st.p0);
        exp_tile8<C>(st, cur, 1, c, st.p1);
      } else {
        st.l32 = lsum;
      }
    }
  }
}

// Step B: O^T = alpha O^T + V^T P^T from V stage VST || row max of the next
// block (first half), then the probabilities of its keys 0..31 (second half).
template <class C, int VST>
__device__ __forceinline__ void step_b8(Fp8State<C>& st, const Scores8<C>& nxt,
                                        const uint8_t XS_LDS* lds, const LdsOffs8<C>& off, float c,
                                        const i32x8& ones) {
  constexpr int DT = C::DT, ROWB = C::ROWB;
  constexpr int NF = DT;
  constexpr int HALF = NF / 2;
  constexpr int LEAD = XS_LEAD8 < NF ? XS_LEAD8 : NF;
  constexpr int R = LEAD + 1;
  if (st.rescale) rescale_o8<C>(st);
  const i32x8 pf = __builtin_bit_cast(
      i32x8, (u32x8{st.p0[0], st.p0[1], st.p0[2], st.p0[3], st.p1[0], st.p1[1], st.p1[2], st.p1[3]}));
  const uint8_t XS_LDS* vb = lds + (C::STAGES + VST) * C::TILE;
  auto vread = [&](int f) {
    u32x2 r[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) r[t] = lds_read_tr8(vb + off.v[f] + 8 * t * ROWB);
    return __builtin_bit_cast(
        i32x8, (u32x8{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]}));
  };
  float mx = C::LSE ? 0.0f : st.mx0;
  float neg_m = 0.0f, lsum = 0.0f, pa = 0.0f, pb = 0.0f;
  uint32_t w[4];
  f32x4 pe[4];
  i32x8 vf[R];
#pragma unroll
  for (int f = 0; f < LEAD; ++f) vf[f] = vread(f);
  if (C::LSE) {
    neg_m = -st.m;
    pa = prob_a<C>(c);
    pb = prob_b<C>(neg_m);
    lsum = st.l32;
    st.lb = st.l32;
  }
  // the micro-step that computes probability group q (keys 4q..4q+3 of each
  // half-wave's 32); it is packed one micro-step later.  Without the log-sum-exp
  // the groups follow the max decision of micro-step 0 (D = 128: groups 0, 1 in
  // micro-step 1, 2 in 2, 3 in 3); with it, one group per micro-step.
  auto at = [&](int q) { return C::LSE ? q * NF / 4 : 1 + q * (NF - 1) / 4; };
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    if (f + LEAD < NF) vf[(f + LEAD) % R] = vread(f + LEAD);
    st.o[f] = mfma_fp8(vf[f % R], pf, st.o[f]);
    if (!C::LSE && f == NF - 1) st.lt = mfma_rowsum(ones, pf, st.lt);
    if (!C::LSE && f == 0) {
      // the rest of the next block's row max and the lazy move of the running
      // max (the O rescale waits for the next step B)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, nxt.s[1][r]);
      const float mnew = max_halves(mx) * c;
      const bool need = mnew > st.m + C::TAU;
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float a = need ? fast_exp2(st.m - mnew) : 1.0f;
        st.m = need ? mnew : st.m;
        st.alpha *= a;
        st.rescale = true;
      }
      neg_m = -st.m;
      pa = prob_a<C>(c);
      pb = prob_b<C>(neg_m);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (f >= 1 && at(q) == f - 1) w[q] = packp4<C>(pe[q]);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (at(q) == f) pe[q] = prob4<C>(nxt, 0, q, pa, pb, lsum);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (at(q) == NF - 1) w[q] = packp4<C>(pe[q]);
  st.l32 = lsum;
  st.p0 = u32x4{w[0], w[1], w[2], w[3]};
  keep(st.p0);
}


// O^T = alpha O^T + V^T P^T (and the row sums) of the last block of a piece,
// from the V stage at byte offset stage_off of the V region (not pipelined).
template <class C>
__device__ __forceinline__ void pv_only8(Fp8State<C>& st, const uint8_t XS_LDS* lds,
                                         const LdsOffs8<C>& off, uint32_t stage_off,
                                         const i32x8& ones) {
  if (st.rescale) rescale_o8<C>(st);
  const i32x8 pf = __builtin_bit_cast(
      i32x8, (u32x8{st.p0[0], st.p0[1], st.p0[2], st.p0[3], st.p1[0], st.p1[1], st.p1[2], st.p1[3]}));
  const uint8_t XS_LDS* vb = lds + C::STAGES * C::TILE + stage_off;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) {
    u32x2 r[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) r[t] = lds_read_tr8(vb + off.v[dt] + 8 * t * C::ROWB);
    const i32x8 vf = __builtin_bit_cast(
        i32x8, (u32x8{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]}));
    st.o[dt] = mfma_fp8(vf, pf, st.o[dt]);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (!C::LSE) st.lt = mfma_rowsum(ones, pf, st.lt);
}

// Takes the next piece of the walk and issues its first loads: K of blocks jb,
// jb+1, jb+2 and V of blocks jb, jb+1 into ring stages 0, 1, 2 (stage of block
// i = (i - jb) % 4).
template <class C>
__device__ __forceinline__ PieceAddr begin_piece8(ShareWalk& walk, const Sched& sch,
                                                  const AttnArgs& a, int nblk, uint32_t row_stride,
                                                  uint8_t XS_LDS* lds,
                                                  const uint32_t (&koff)[C::LPW],
                                                  const uint32_t (&voff)[C::LPW], int wave,
                                                  int& slot) {
  PieceAddr pa = next_piece<C::BM, C::ROWB, C::BN>(walk, sch, a, nblk, row_stride, slot);
  const uint8_t* kbase = (const uint8_t*)a.k + pa.head_off;
  const uint8_t* vbase = (const uint8_t*)a.v + pa.head_off;
  uint8_t XS_LDS* const vlds = lds + C::STAGES * C::TILE;
  load_tile8<C>(kbase, row_stride, pa.jb * C::BN, pa.kcur.at(pa.jb), a.S, lds, koff, wave);
  load_tile8<C>(vbase, row_stride, pa.jb * C::BN, pa.vcur.at(pa.jb), a.S, vlds, voff, wave);
  if (pa.jb + 1 < pa.je) {
    load_tile8<C>(kbase, row_stride, (pa.jb + 1) * C::BN, pa.kcur.at(pa.jb + 1), a.S,
                  lds + C::TILE, koff, wave);
    load_tile8<C>(vbase, row_stride, (pa.jb + 1) * C::BN, pa.vcur.at(pa.jb + 1), a.S,
                  vlds + C::TILE, voff, wave);
  }
  if (pa.jb + 2 < pa.je)
    load_tile8<C>(kbase, row_stride, (pa.jb + 2) * C::BN, pa.kcur.at(pa.jb + 2), a.S,
                  lds + 2 * C::TILE, koff, wave);
  return pa;
}

// Loads the piece's query rows (clamped to the sequence) as Q^T B-operand
// fragments, negated when the scale is negative.
template <class C>
__device__ __forceinline__ void load_q8(i32x8 (&qf)[C::KS], const AttnArgs& a, const PieceAddr& pa,
                                        uint32_t row_stride, uint32_t qflip, int wave, int lane) {
  int qrow = pa.m0 + wave * C::QW + (lane & 31);
  qrow = qrow < a.S ? qrow : a.S - 1;
  const long long qr = qrow + (a.chunk_rows ? (long long)(qrow / a.chunk_rows) * a.jump_rows : 0);
  const uint8_t* qp = (const uint8_t*)a.q + pa.head_off + (size_t)qr * row_stride + (lane >> 5) * 32;
#pragma unroll
  for (int t = 0; t < C::KS; ++t) {
    const u32x4 x0 = *(const u32x4*)(qp + t * 64) ^ qflip;
    const u32x4 x1 = *(const u32x4*)(qp + t * 64 + 16) ^ qflip;
    qf[t] = __builtin_bit_cast(i32x8, (u32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]}));
  }
}

// Persistent workgroups walking their chunk of the schedule piece by piece, as
// in the bf16 kernel (attn_fwd_bf16.hip).
template <class C>
__global__ __launch_bounds__(C::THREADS, 1) void attn_fwd_fp8_kernel(AttnArgs a) {
  constexpr int BN = C::BN;
  // K stages 0..3 | V stages 0..3
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * C::STAGES * C::TILE];
  uint8_t XS_LDS* const lds = (uint8_t XS_LDS*)smem;
  auto kbuf = [&](int s) { return lds + s * C::TILE; };
  auto vbuf = [&](int s) { return lds + (C::STAGES + s) * C::TILE; };

  const int S = a.S, H = a.H, T = a.T, B = a.B;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const uint32_t row_stride = (uint32_t)H * C::ROWB;
  // this lane's 16-byte chunk of each of the wave's 1 KiB direct loads, for K and V
  uint32_t koff[C::LPW], voff[C::LPW];
  if constexpr (C::LPW == 1) {
    const int pos = wave * 64 + lane;
    const int R = pos / C::CH, cp = pos % C::CH;
    koff[0] = (uint32_t)R * row_stride + (uint32_t)((cp ^ kswz<C>(R)) * 16);
    voff[0] = (uint32_t)vrow_key(R) * row_stride + (uint32_t)((cp ^ vswz<C>(R)) * 16);
  } else {
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) {
      const int pos = (wave * C::LPW + i) * 64 + lane;
      const int R = pos / C::CH, cp = pos % C::CH;
      koff[i] = (uint32_t)R * row_stride + (uint32_t)((cp ^ kswz<C>(R)) * 16);
      voff[i] = (uint32_t)vrow_key(R) * row_stride + (uint32_t)((cp ^ vswz<C>(R)) * 16);
    }
  }
  const int nblk = (S + BN - 1) / BN;
  const int nfull = S / BN;
  const uint32_t qflip = a.neg ? 0x80808080u : 0u;
  const float c = a.c;
  const LdsOffs8<C> off = lds_offsets8<C>(lane);
  // the row-sum MFMA's constant operand, held in registers for the whole kernel
  // (opaque, so the compiler does not rebuild it before every use)
  i32x8 ones = ones_e4m3(lane);
  asm volatile("" : "+v"(ones));

  const Sched sch{a.units, a.groups, a.npair, a.dp};
  ShareWalk walk;
  walk.init(sch, xcd_tile(blockIdx.x, a.groups));
  if (!walk.more(sch)) return;
  int slot;
  PieceAddr pa = begin_piece8<C>(walk, sch, a, nblk, row_stride, lds, koff, voff, wave, slot);
  Fp8State<C> st;
  load_q8<C>(st.qf, a, pa, row_stride, qflip, wave, lane);

  for (;;) {
    const int jb = pa.jb, je = pa.je, m0 = pa.m0;
    const uint8_t* kbase = (const uint8_t*)a.k + pa.head_off;
    const uint8_t* vbase = (const uint8_t*)a.v + pa.head_off;

    st.m = -INFINITY;
    st.lt = f32x4{};
    st.l32 = 0.0f;
    st.alpha = 1.0f;
    st.rescale = false;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) st.o[dt] = f32x16{};

    wait_vmcnt<0>();
    __syncthreads();

    // prologue: score block jb, take its max, probabilities of its keys 0..31
    Scores8<C> sa, sb;
    qk_block8<C>(sa, st, kbuf(0), lane);
    if (jb >= nfull) mask_tail8<C>(sa, jb * BN, S, lane);
    softmax_max8<C>(st, sa, c);
    st.lb = st.l32;
    exp_tile8<C>(st, sa, 0, c, st.p0);

    // K/V blocks stream through a four-stage LDS ring with one barrier per two
    // blocks, as in the bf16 kernel: at the barrier before blocks i, i+1
    // (i - jb even) the loads of K_{i+1}, K_{i+2}, V_i, V_{i+1} are complete
    // and blocks i-2, i-1 are done, so K_{i+3}, K_{i+4}, V_{i+2}, V_{i+3} go
    // into their stages, one before each of the next four steps (1.2 % faster
    // than all four at the barrier).  Entering a step for block i: its scores
    // are in one buffer with their max taken and the probabilities of keys
    // 0..31 in st.p0.
    auto ld_k = [&](int i, int stage) {
      load_tile8<C>(kbase, row_stride, i * BN, pa.kcur.at(i), S, kbuf(stage), koff, wave);
    };
    auto ld_v = [&](int i, int stage) {
      load_tile8<C>(vbase, row_stride, i * BN, pa.vcur.at(i), S, vbuf(stage), voff, wave);
    };
    int j = jb;
    for (; j + 4 < je; j += 4) {
      wait_vmcnt<0>();
      __syncthreads();
      ld_k(j + 3, 3);
      step_a8<C, 1>(sb, sa, st, lds, off, c);  // block j
      if (j + 1 >= nfull) mask_tail_next8<C>(sb, st, (j + 1) * BN, S, lane);
      ld_v(j + 2, 2);
      step_b8<C, 0>(st, sb, lds, off, c, ones);
      ld_k(j + 4, 0);
      step_a8<C, 2>(sa, sb, st, lds, off, c);  // block j+1
      if (j + 2 >= nfull) mask_tail_next8<C>(sa, st, (j + 2) * BN, S, lane);
      ld_v(j + 3, 3);
      step_b8<C, 1>(st, sa, lds, off, c, ones);

      wait_vmcnt<0>();
      __syncthreads();
      if (j + 5 < je) ld_k(j + 5, 1);
      step_a8<C, 3>(sb, sa, st, lds, off, c);  // block j+2
      if (j + 3 >= nfull) mask_tail_next8<C>(sb, st, (j + 3) * BN, S, lane);
      ld_v(j + 4, 0);
      step_b8<C, 2>(st, sb, lds, off, c, ones);
      if (j + 6 < je) ld_k(j + 6, 2);
      step_a8<C, 0>(sa, sb, st, lds, off, c);  // block j+3
      if (j + 4 >= nfull) mask_tail_next8<C>(sa, st, (j + 4) * BN, S, lane);
      if (j + 5 < je) ld_v(j + 5, 1);
      step_b8<C, 3>(st, sa, lds, off, c, ones);
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
        step_a8<C, 1>(sb, sa, st, lds, off, c);  // block j
        if (j + 1 >= nfull) mask_tail_next8<C>(sb, st, (j + 1) * BN, S, lane);
        step_b8<C, 0>(st, sb, lds, off, c, ones);
      }
      if (r > 2) {
        step_a8<C, 2>(sa, sb, st, lds, off, c);  // block j+1
        if (j + 2 >= nfull) mask_tail_next8<C>(sa, st, (j + 2) * BN, S, lane);
        step_b8<C, 1>(st, sa, lds, off, c, ones);
        wait_vmcnt<0>();
        __syncthreads();
      }
      if (r > 3) {
        step_a8<C, 3>(sb, sa, st, lds, off, c);  // block j+2
        if (j + 3 >= nfull) mask_tail_next8<C>(sb, st, (j + 3) * BN, S, lane);
        step_b8<C, 2>(st, sb, lds, off, c, ones);
      }
      // the last block, j + r - 1: scores in sa when r is odd, keys 0..31 done
      if (C::LSE) {
        // its max not yet taken: take it, then recompute all its probabilities
        st.l32 = st.lb;
        if (r & 1) {
          softmax_max8<C>(st, sa, c);
          exp_tile8<C>(st, sa, 0, c, st.p0);
          exp_tile8<C>(st, sa, 1, c, st.p1);
        } else {
          softmax_max8<C>(st, sb, c);
          exp_tile8<C>(st, sb, 0, c, st.p0);
          exp_tile8<C>(st, sb, 1, c, st.p1);
        }
      } else if (r & 1) {
        exp_tile8<C>(st, sa, 1, c, st.p1);
      } else {
        exp_tile8<C>(st, sb, 1, c, st.p1);
      }
      pv_only8<C>(st, lds, off, (uint32_t)(r - 1) * C::TILE, ones);
    }

    // ---- next piece: request its first K/V blocks and its queries before
    // this piece's stores
    const bool more = walk.more(sch);
    const PieceAddr cur = pa;
    const int cur_slot = slot;
    if (more) {
      __syncthreads();  // every wave is done reading this piece's tiles
      pa = begin_piece8<C>(walk, sch, a, nblk, row_stride, lds, koff, voff, wave, slot);
      load_q8<C>(st.qf, a, pa, row_stride, qflip, wave, lane);
    }

    // ---- epilogue
    const int srow = m0 + wave * C::QW + (lane & 31);
    if (cur.whole) {
      // O * dv / l, rounded to bf16, stored into the destination slice
      const float lrow = row_sum(st);
      const float inv = a.o_scale / lrow;
      if (C::LSE && lane < 32 && srow < S) a.lse[(size_t)cur.bh * S + srow] = row_lse(st.m, lrow);
      if (srow < S) {
        const int p = srow / T;
        const int sp = srow - p * T;
        uint16_t* orow = (uint16_t*)a.out + ((((size_t)p * B + cur.b) * T + sp) * H + cur.h) * C::D;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int d0 = dt * 32 + r4 * 8 + 4 * (lane >> 5);
            const f32x16& o = st.o[dt];
            u32x2 w = {pack_bf16(o[4 * r4 + 0] * inv, o[4 * r4 + 1] * inv),
                       pack_bf16(o[4 * r4 + 2] * inv, o[4 * r4 + 3] * inv)};
            *(u32x2*)(orow + d0) = w;
          }
      }
    } else {
      // a tile cut between shares: fp32 partials into this share's slot, O in
      // register order as in the bf16 kernel (1 KiB per store instruction)
      const float lsum = row_sum(st);
      const int r = srow - m0;
      if (srow < S) {
        const size_t sr = (size_t)cur_slot * C::BM + r;
        float* og = a.ws_o + ((size_t)cur_slot * C::BM + wave * C::QW) * C::D;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const f32x16& o = st.o[dt];
            *(f32x4*)(og + ((dt * 4 + r4) * 64 + lane) * 4) =
                f32x4{o[4 * r4 + 0], o[4 * r4 + 1], o[4 * r4 + 2], o[4 * r4 + 3]};
          }
        if (lane < 32) *(f32x2*)(a.ws_ml + 2 * sr) = f32x2{st.m, lsum};
      }
    }
    if (!more) break;
  }
}

template <class C>
static hipError_t launch_cfg8(const AttnArgs& a, hipStream_t stream) {
  if (a.groups < 1) return hipErrorInvalidValue;
  AttnArgs args = a;
  void* kargs[] = {&args};
  return hipLaunchKernel((const void*)attn_fwd_fp8_kernel<C>, dim3((unsigned)a.groups),
                         dim3(C::THREADS), kargs, 0, stream);
}

// Full-height tiles (8 waves), or half-height ones (4 waves) for the tiles a
// call without cut tiles leaves after its whole rounds; half tiles are never cut.
template <int D, bool LSE>
static hipError_t launch_d8(const AttnArgs& a, hipStream_t stream) {
  using C = Fp8Cfg<D, LSE>;
  using CH = Fp8Cfg<D, LSE, 4>;
  static_assert(C::BM == kBlockM && C::BN == kBlockN, "tile geometry");
  static_assert(CH::BM == kHalfM && CH::BN == kBlockN, "tile geometry");
  if (!a.half) return launch_cfg8<C>(a, stream);
  if (a.ws_o != nullptr || a.units != 0) return hipErrorInvalidValue;
  return launch_cfg8<CH>(a, stream);
}

hipError_t launch_attn_fp8(const AttnArgs& a, hipStream_t stream) {
  switch (a.D) {
    case 64:
      return a.lse ? launch_d8<64, true>(a, stream) : launch_d8<64, false>(a, stream);
    case 128:
      return a.lse ? launch_d8<128, true>(a, stream) : launch_d8<128, false>(a, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace xs
