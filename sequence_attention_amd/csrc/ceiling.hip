// ceiling.hip -- matrix-core ceiling probes: v_mfma_f32_32x32x16_bf16 issued
// back to back next to the LDS operand reads and the softmax vector work of
// the attention kernels (declared in xs_ceiling.h).
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "xs_ceiling.h"

namespace xs {
namespace {

constexpr int kInner = 16;                    // MFMAs per loop trip
constexpr int kLead = 3;                      // LDS reads issued this many MFMAs ahead
constexpr int kGroups = 1024;

__device__ __forceinline__ f32x4 mfma16_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                 c, 0, 0, 0);
}

// Two N(0, 1) draws for LDS word i of the data modes (Box-Muller on a hash of
// i): the workloads' inputs are N(0, 1) draws.
__device__ __forceinline__ f32x2 normal_pair(uint32_t i) {
  uint32_t h = i * 2654435761u;
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 12;
  const uint32_t g = (h ^ 0x5bd1e995u) * 0x9E3779B1u;
  const float u1 = ((h >> 8) + 1u) * (1.0f / 16777217.0f);  // (0, 1]
  const float u2 = (g >> 8) * (1.0f / 16777216.0f);
  const float r = __builtin_sqrtf(-2.0f * __logf(u1));
  return f32x2{r * __cosf(6.2831853f * u2), r * __sinf(6.2831853f * u2)};
}

// LDS word i of the bf16 data modes: two N(0, 1) values as bf16 (truncated);
// read as an fp32 the word is its upper value with noise in the low mantissa bits.
__device__ __forceinline__ uint32_t data_word(uint32_t i) {
  const f32x2 n = normal_pair(i);
  return (__float_as_uint(n[0]) & 0xFFFF0000u) | (__float_as_uint(n[1]) >> 16);
}

// One trip's worth of a mode's extra stream is written out per MFMA; the
// scheduling barrier after each MFMA and its slice keeps the interleave.
template <int MODE, int THREADS>
__global__ __launch_bounds__(THREADS, 1) void ceiling_kernel(float* sink, int iters) {
  // 96 KiB: one workgroup per compute unit; reads stay below 68 KiB of it
  __shared__ __attribute__((aligned(1024))) uint8_t smem[96 * 1024];
  uint8_t XS_LDS* lds = (uint8_t XS_LDS*)smem;
  const int lane = threadIdx.x & 63;
  constexpr bool kData = MODE == XS_CEIL_MFMA_DATA || MODE == XS_CEIL_MIX_DATA || MODE == XS_CEIL_MFMA16_DATA ||
                        MODE == XS_CEIL_MIX16_DATA;
  constexpr bool k16 = MODE == XS_CEIL_MFMA16_DATA || MODE == XS_CEIL_MIX16_DATA;
  constexpr bool kRegf = MODE == XS_CEIL_MFMA_DATA || MODE == XS_CEIL_MFMA16_DATA;
  for (uint32_t i = threadIdx.x * 4; i < sizeof(smem); i += THREADS * 4)
    *(uint32_t XS_LDS*)(lds + i) = kData ? data_word(i >> 2) : i * 2654435761u;
  __syncthreads();

  constexpr bool kPerMfma = MODE == XS_CEIL_LDS_1K || MODE == XS_CEIL_TR16_1K || MODE == XS_CEIL_MIX ||
                           MODE == XS_CEIL_MIX_DATA || MODE == XS_CEIL_MIX16_DATA;
  constexpr bool kHalf = MODE == XS_CEIL_LDS_HALF || MODE == XS_CEIL_MIX_HALF;
  constexpr bool kSoftmax = MODE == XS_CEIL_SOFTMAX || MODE == XS_CEIL_MIX || MODE == XS_CEIL_MIX_HALF ||
                           MODE == XS_CEIL_MIX_DATA || MODE == XS_CEIL_MIX16_DATA;
  f32x16 acc[4] = {};
  f32x4 acc16[8] = {};
  const u32x4 a = {lane * 3u, lane * 5u, 7u, 9u};
  // softmax stand-in, as in the bf16 kernel: p = 2^(x c - m) of eight independent
  // chains, their row sum, and the pairs rounded to bf16 as the next MFMAs' B operand
  float z[8], lsum = 0.0f;
  uint32_t pk[4] = {lane * 11u, 13u, 17u, 19u};
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = 0.5f + lane * 0.001f + 0.01f * i;
  // one fragment per 1 KiB of a 16 KiB window per loop trip, the window moving by
  // 16 KiB per trip over four positions: offsets are immediates within a trip
  u32x4 frag[kLead + 1];
  auto read = [&](const uint8_t XS_LDS* tb, int f) -> u32x4 {
    if (MODE == XS_CEIL_TR16_1K) {
      const u32x2 lo = lds_read_tr16(tb + f * 1024);
      const u32x2 hi = lds_read_tr16(tb + f * 1024 + 512);
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
    return lds_read_b128(tb + f * 1024);
  };
  const uint8_t XS_LDS* const lane_base = lds + (MODE == XS_CEIL_TR16_1K ? lane * 8 : lane * 16);
  // MFMAs-only data mode: eight register-held fragments of the LDS data, A and B
  // rotating through them so that every MFMA sees new operand bits
  u32x4 regf[8];
  if (kRegf)
#pragma unroll
    for (int i = 0; i < 8; ++i) regf[i] = lds_read_b128(lane_base + i * 1024);
  if (kPerMfma || kHalf)
#pragma unroll
    for (int k = 0; k < kLead; ++k) frag[k] = read(lane_base, k);

  for (int it = 0; it < iters; ++it) {
    const uint8_t XS_LDS* tb = lane_base + (it & 3) * 16384;
#pragma unroll
    for (int k = 0; k < kInner; ++k) {
      u32x4 op = a;
      u32x4 opb = u32x4{pk[0], pk[1], pk[2], pk[3]};
      if (kRegf) {
        op = regf[k & 7];
        opb = regf[(k + 3) & 7];
      } else if (kPerMfma) {
        frag[(k + kLead) % (kLead + 1)] = read(tb, k + kLead);
        op = frag[k % (kLead + 1)];
      } else if (kHalf) {
        if ((k & 1) == 0) frag[((k >> 1) + kLead) % (kLead + 1)] = read(tb, (k >> 1) + kLead);
        op = frag[(k >> 1) % (kLead + 1)];
      }
      if (MODE == XS_CEIL_MFMA16_DATA) {
        // the same multiply-adds as one 32x32x16 MFMA, as two 16x16x32 ones
        acc16[(2 * k) & 7] = mfma16_bf16(op, opb, acc16[(2 * k) & 7]);
        acc16[(2 * k + 1) & 7] = mfma16_bf16(regf[(k + 1) & 7], opb, acc16[(2 * k + 1) & 7]);
      } else if (MODE == XS_CEIL_MIX16_DATA) {
        // one LDS fragment as the A operand of two 16x16x32 MFMAs (two 16-query
        // tiles); the second B operand is the next MFMA's fragment (random data
        // already in registers)
        acc16[(2 * k) & 7] = mfma16_bf16(op, opb, acc16[(2 * k) & 7]);
        acc16[(2 * k + 1) & 7] = mfma16_bf16(op, frag[(k + 1) % (kLead + 1)], acc16[(2 * k + 1) & 7]);
      } else {
        acc[k & 3] = mfma_bf16(op, opb, acc[k & 3]);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (kSoftmax) {
        // data mode: the exponent's argument is a new value each time (this MFMA's
        // A word read as fp32, an N(0, 1) draw), scaled as the video share's scores
        // relative to the running max: x·1.44 - 5, so p = 2^-5 typically, 2^-10 .. 1
        const float x = kData ? __uint_as_float(op[k & 3]) : z[k & 7];
        z[k & 7] = kData ? __builtin_amdgcn_exp2f(__builtin_fmaf(x, 1.44f, -5.0f))
                         : __builtin_amdgcn_exp2f(__builtin_fmaf(x, 0.5f, -0.4f));
        lsum += z[k & 7];
        if (k & 1) pk[(k >> 1) & 3] = pack_bf16(z[(k - 1) & 7], z[k & 7]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  float s = lsum;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[q][r];
#pragma unroll
  for (int i = 0; i < 8; ++i) s += z[i];
  if (kPerMfma || kHalf)
#pragma unroll
    for (int k = 0; k <= kLead; ++k) s += (float)(frag[k][0] ^ frag[k][3]);
  if (kRegf)
#pragma unroll
    for (int k = 0; k < 8; ++k) s += (float)(regf[k][1] & 0xFFu);
  if (k16)
#pragma unroll
    for (int k = 0; k < 8; ++k) s += acc16[k][0] + acc16[k][3];
  sink[blockIdx.x * 512 + threadIdx.x] = s;
}


// The fp8 modes: v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 x e4m3, 64 clocks, four
// times the multiply-adds of a bf16 32x32x16) on e4m3 data like the fp8
// workload's.  XS_CEIL_FP8_DATA: A and B rotate through eight register-held
// 32-byte fragments.  XS_CEIL_FP8_MIX_DATA: the fp8 attention kernel's per-MFMA
// work -- 2 KiB of LDS operand (two ds_read_b128, read three MFMAs ahead) as A,
// and as B the e4m3 codes of its probabilities: per MFMA four FMAs, two
// normalised 16-bit conversions, one byte permutation (and a mask that keeps the
// codes below the NaN code, one instruction the kernel does not need) and two
// three-input maxima on scores from the accumulator two MFMAs back.
template <int MODE, int THREADS>
__global__ __launch_bounds__(THREADS, 1) void ceiling_fp8_kernel(float* sink, int iters) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[96 * 1024];
  uint8_t XS_LDS* lds = (uint8_t XS_LDS*)smem;
  const int lane = threadIdx.x & 63;
  // four N(0, 1) draws per word quantised as the fp8 workload's inputs are:
  // e4m3 (round to nearest even) of x / (amax / 448) with amax = 5
  for (uint32_t i = threadIdx.x * 4; i < sizeof(smem); i += THREADS * 4) {
    const f32x2 n0 = normal_pair(2 * (i >> 2)), n1 = normal_pair(2 * (i >> 2) + 1);
    constexpr float q = 448.0f / 5.0f;
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(n0[0] * q, n0[1] * q, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(n1[0] * q, n1[1] * q, w, true);
    *(uint32_t XS_LDS*)(lds + i) = (uint32_t)w;
  }
  __syncthreads();
  constexpr bool kMix = MODE == XS_CEIL_FP8_MIX_DATA;
  const uint8_t XS_LDS* const lane_base = lds + lane * 16;
  auto read = [&](const uint8_t XS_LDS* tb, int f) -> i32x8 {
    const u32x4 a0 = lds_read_b128(tb + f * 2048);
    const u32x4 a1 = lds_read_b128(tb + f * 2048 + 1024);
    return __builtin_bit_cast(i32x8, (u32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]}));
  };
  f32x16 acc[4] = {};
  i32x8 regf[8];
  i32x8 frag[kLead + 1];
  uint32_t code[8];
  float mx = 0.0f;
  if (!kMix) {
#pragma unroll
    for (int i = 0; i < 8; ++i) regf[i] = read(lane_base, i);
  } else {
#pragma unroll
    for (int k = 0; k < kLead; ++k) frag[k] = read(lane_base, k);
#pragma unroll
    for (int i = 0; i < 8; ++i) code[i] = (uint32_t)read(lane_base, 8 + i)[0] & 0x7E7E7E7Eu;
  }
  for (int it = 0; it < iters; ++it) {
    const uint8_t XS_LDS* tb = lane_base + (it & 1) * 32768;
#pragma unroll
    for (int k = 0; k < kInner; ++k) {
      i32x8 a, b;
      if (!kMix) {
        a = regf[k & 7];
        b = regf[(k + 3) & 7];
      } else {
        frag[(k + kLead) % (kLead + 1)] = read(tb, k + kLead);
        a = frag[k % (kLead + 1)];
        b = __builtin_bit_cast(i32x8, (u32x8{code[0], code[1], code[2], code[3], code[4], code[5], code[6], code[7]}));
      }
      // the mix restarts each accumulator every second use, as the kernel's score
      // tiles start every block (D = 128: two k-steps), so its values stay in range
      acc[k & 3] = mfma_fp8(a, b, (!kMix || (k & 4)) ? acc[k & 3] : f32x16{});
      __builtin_amdgcn_sched_barrier(0);
      if (kMix) {
        const f32x16& sc = acc[(k + 2) & 3];  // written two MFMAs back
        float t[4];
#pragma unroll
        // codes 8 (x - m + 11.75) of the fp8 share's scores (x - m = -5 +- 1.44
        // typically: codes near 54 +- 12) from the accumulator's values: sums of
        // 128 products of two e4m3 draws of standard deviation 89.6, +-9.1e4
        for (int i = 0; i < 4; ++i)
          t[i] = __builtin_fmaf(sc[4 * (k & 3) + i], 12.0f / (9.1e4f * 65535.0f), 54.0f / 65535.0f);
        mx = fmaxf(fmaxf(mx, sc[4 * (k & 3)]), sc[4 * (k & 3) + 1]);
        mx = fmaxf(fmaxf(mx, sc[4 * (k & 3) + 2]), sc[4 * (k & 3) + 3]);
        const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pknorm_u16(t[0], t[1]));
        const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pknorm_u16(t[2], t[3]));
        code[k & 7] = __builtin_amdgcn_perm(hi, lo, 0x06040200u) & 0x7E7E7E7Eu;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  float s = mx;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[q][r];
#pragma unroll
  for (int i = 0; i < 8; ++i) s += kMix ? (float)(code[i] & 0xFFu) : (float)(regf[i][1] & 0xFF);
  if (kMix)
#pragma unroll
    for (int k = 0; k <= kLead; ++k) s += (float)(frag[k][0] & 0xFF);
  sink[blockIdx.x * 512 + threadIdx.x] = s;
}

template <int MODE>
hipError_t launch_mode(int waves, float* sink, int iters, hipStream_t stream) {
  if (MODE == XS_CEIL_FP8_DATA || MODE == XS_CEIL_FP8_MIX_DATA) {
    if (waves == 1)
      hipLaunchKernelGGL((ceiling_fp8_kernel<MODE, 256>), dim3(kGroups), dim3(256), 0, stream, sink, iters);
    else
      hipLaunchKernelGGL((ceiling_fp8_kernel<MODE, 512>), dim3(kGroups), dim3(512), 0, stream, sink, iters);
    return hipGetLastError();
  }
  if (waves == 1) {
    hipLaunchKernelGGL((ceiling_kernel<MODE, 256>), dim3(kGroups), dim3(256), 0, stream, sink, iters);
  } else {
    hipLaunchKernelGGL((ceiling_kernel<MODE, 512>), dim3(kGroups), dim3(512), 0, stream, sink, iters);
  }
  return hipGetLastError();
}

// One wave per workgroup: the counters of the compute unit it runs on.  XCC_ID
// is hardware register 20 (bits 3:0 the XCC), HW_ID register 4.
__global__ __launch_bounds__(64) void clock_kernel(unsigned long long* out) {
  if (threadIdx.x != 0) return;
  const unsigned long long t = __builtin_amdgcn_s_memtime();
  const unsigned long long r = __builtin_amdgcn_s_memrealtime();
  const unsigned xcc = __builtin_amdgcn_s_getreg(20 | (3 << 11)) & 0xFu;
  const unsigned hw = __builtin_amdgcn_s_getreg(4 | (31 << 11));
  unsigned long long* o = out + 4 * blockIdx.x;
  o[0] = t;
  o[1] = r;
  o[2] = xcc;
  o[3] = hw;
}

}  // namespace
}  // namespace xs

extern "C" int xs_mfma_ceiling(int mode, int waves_per_simd, int iters, float* sink, size_t sink_bytes,
                               void* stream) {
  using namespace xs;
  if (!sink) return XS_CEIL_ERR_NULL;
  if (mode < 0 || mode >= XS_CEIL_MODES || (waves_per_simd != 1 && waves_per_simd != 2) || iters < 1 ||
      iters > (1 << 20))
    return XS_CEIL_ERR_ARG;
  if (sink_bytes < XS_CEIL_SINK_BYTES) return XS_CEIL_ERR_SIZE;
  if ((uintptr_t)sink % 4) return XS_CEIL_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  switch (mode) {
    case XS_CEIL_MFMA: e = launch_mode<XS_CEIL_MFMA>(waves_per_simd, sink, iters, s); break;
    case XS_CEIL_LDS_1K: e = launch_mode<XS_CEIL_LDS_1K>(waves_per_simd, sink, iters, s); break;
    case XS_CEIL_LDS_HALF: e = launch_mode<XS_CEIL_LDS_HALF>(waves_per_simd, sink, iters, s); break;
    case XS_CEIL_TR16_1K: e = launch_mode<XS_CEIL_TR16_1K>(waves_per_simd, sink, iters, s); break;
    case XS_CEIL_SOFTMAX: e = launch_mode<XS_CEIL_SOFTMAX>(waves_per_simd, sink, iters, s); break;
    case XS_CEIL_MIX: e = launch_mode<XS_CEIL_MIX>(waves_per_simd, sink, iters, s); break;
    case XS_CEIL_MIX_HALF: e = launch_mode<XS_CEIL_MIX_HALF>(waves_per_simd, sink, iters, s); break;
    case XS_CEIL_MFMA_DATA: e = launch_mode<XS_CEIL_MFMA_DATA>(waves_per_simd, sink, iters, s); break;
    case XS_CEIL_MFMA16_DATA: e = launch_mode<XS_CEIL_MFMA16_DATA>(waves_per_simd, sink, iters, s); break;
    case XS_CEIL_MIX16_DATA: e = launch_mode<XS_CEIL_MIX16_DATA>(waves_per_simd, sink, iters, s); break;
    case XS_CEIL_FP8_DATA: e = launch_mode<XS_CEIL_FP8_DATA>(waves_per_simd, sink, iters, s); break;
    case XS_CEIL_FP8_MIX_DATA: e = launch_mode<XS_CEIL_FP8_MIX_DATA>(waves_per_simd, sink, iters, s); break;
    default: e = launch_mode<XS_CEIL_MIX_DATA>(waves_per_simd, sink, iters, s); break;
  }
  return e == hipSuccess ? 0 : XS_CEIL_ERR_LAUNCH;
}

extern "C" int xs_clock_sample(unsigned long long* out, size_t out_bytes, int* wall_khz, void* stream) {
  using namespace xs;
  if (!out || !wall_khz) return XS_CEIL_ERR_NULL;
  if (out_bytes < XS_CLOCK_BYTES) return XS_CEIL_ERR_SIZE;
  if ((uintptr_t)out % 8) return XS_CEIL_ERR_ALIGN;
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
    return XS_CEIL_ERR_LAUNCH;
  *wall_khz = khz;
  hipLaunchKernelGGL(clock_kernel, dim3(XS_CLOCK_GROUPS), dim3(64), 0, (hipStream_t)stream, out);
  return hipGetLastError() == hipSuccess ? 0 : XS_CEIL_ERR_LAUNCH;
}
