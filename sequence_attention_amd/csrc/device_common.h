// device_common.h -- small gfx950 device helpers shared by the attention
// kernels: vector types, MFMA wrappers, LDS transpose reads, direct-to-LDS
// loads, cross-half-wave reductions and the XCD-aware tile order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

#define XS_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;

// D(32x32 fp32) += A(32x16 bf16) * B(16x32 bf16).  Lane l supplies row l%32 of
// A and column l%32 of B, eight consecutive k values starting at 8*(l/32).
// The result element (row, col) sits in lane col + 32*((row/4)%2), register
// (row/8)*4 + row%4.
__device__ __forceinline__ f32x16 mfma_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// D(32x32 fp32) += A(32x64 e4m3) * B(64x32 e4m3); lane l holds 32 consecutive
// k values starting at 32*(l/32) of row/column l%32.
__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane j receives element
// j%4 of the 64-bit words addressed by lanes 4e + j/4, e = 0..3.  When lane L
// of the group addresses row r0 + L/4, columns c0 + 4*(L%4) .. +3 of a
// row-major 16-bit matrix, lane j receives rows r0..r0+3 of column c0 + j.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint8_t XS_LDS* p) {
  i16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 XS_LDS*)p);
  return __builtin_bit_cast(u32x2, t);
}

// ds_read_b64_tr_b8: within each group of 16 lanes, lane j receives byte j%8
// of the 64-bit words addressed by lanes 2e + j/8, e = 0..7.  When lane L of
// the group addresses row r0 + L/2, columns c0 + 8*(L%2) .. +7 of a row-major
// byte matrix, lane j receives rows r0..r0+7 of column c0 + j.
__device__ __forceinline__ u32x2 lds_read_tr8(const uint8_t XS_LDS* p) {
  typedef int i32x2 __attribute__((ext_vector_type(2)));
  i32x2 t = __builtin_amdgcn_ds_read_tr8_b64_v2i32((i32x2 XS_LDS*)p);
  return __builtin_bit_cast(u32x2, t);
}

__device__ __forceinline__ u32x4 lds_read_b128(const uint8_t XS_LDS* p) {
  return *(const u32x4 XS_LDS*)p;
}

// Raw buffer resource (stride 0) over `bytes` bytes from `base`; buffer loads
// at offsets past `bytes` return zeros instead of touching memory.
__device__ __forceinline__ u32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, bytes, 0x00020000u};
}

// One direct-to-LDS 16-byte buffer load per lane: the 16 bytes at byte offset
// `voff` of the resource land at LDS address lds_addr + 16*lane (lds_addr
// wave-uniform).  Written as inline asm so the compiler does not order its own
// LDS reads behind these loads: completion is tracked explicitly with
// wait_vmcnt + a workgroup barrier before the tile is read.  The instruction
// has no VGPR result, and its address VGPR is consumed at issue.
__device__ __forceinline__ void load_lds_b128(u32x4 rsrc, uint32_t voff, uint32_t lds_addr) {
  // M0 holds the LDS destination base; the compiler writes it (the "{m0}"
  // operand), the s_nop covers the M0-write to LDS-DMA distance.
  asm volatile(
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(rsrc), "{m0}"(lds_addr)
      : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const uint8_t XS_LDS* p) {
  return (uint32_t)(uintptr_t)p;
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Both halves of a value held by lanes l and l^32: returns {x[l%32], x[l%32+32]}
// in some order, so max/sum of the pair is the reduction over the two halves.
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Two fp32 values -> packed bf16 pair (round to nearest even), low half first.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Natural-log log-sum-exp of a row from its running max m (log2 units) and
// its sum l of 2^(s c - m): ln(2^m l) = (m + log2 l) ln 2.
__device__ __forceinline__ float row_lse(float m, float l) {
  return (m + __builtin_amdgcn_logf(l)) * 0.6931471805599453f;
}

// Marks x as used here: keeps the optimiser from sinking the instructions that
// compute x past this point (into a later block of the software pipeline).
template <class T>
__device__ __forceinline__ void keep(const T& x) {
  asm volatile("" : : "v"(x));
}

// Pins the computation of x to this point of the instruction stream: x must be
// complete here and is opaque afterwards.  Used to place slices of the vector
// work between the matrix instructions of a software-pipelined step.
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(uint32_t& x) { asm volatile("" : "+v"(x)); }

// Returns x unchanged but opaque to the optimiser, so address arithmetic that
// depends on it is recomputed where it is used instead of being hoisted out of
// the loop and kept live (or spilled) across the whole kernel.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Bytes to add to the K/V rows of 64-key block n when the inputs arrive in the
// chunk layout [P][B][T][H][D] (T a multiple of 64): each chunk boundary skips
// the (B-1)*T rows of the other batches.  One stream (K or V) loads its blocks
// in increasing order, one at a time, so a boundary test per load replaces a
// division.  All members are wave-uniform.
struct ChunkCursor {
  int nb;       // first block of the next chunk
  int tpc;      // blocks per chunk
  size_t step;  // bytes skipped at a chunk boundary
  size_t ex;    // bytes skipped before the current chunk
  __device__ void init(int first_block, int chunk_rows, long long jump_rows, uint32_t row_stride) {
    if (chunk_rows == 0) {  // [B][S][H][D]: rows are contiguous
      nb = 0x7fffffff, tpc = 1, step = 0, ex = 0;
      return;
    }
    tpc = chunk_rows / 64;
    const int p = first_block / tpc;
    step = (size_t)jump_rows * row_stride;
    nb = (p + 1) * tpc;
    ex = (size_t)p * step;
  }
  // n must not decrease from one call to the next
  __device__ size_t at(int n) {
    while (n >= nb) {
      nb += tpc;
      ex += step;
    }
    return ex;
  }
};

// Workgroups are dispatched round-robin over the 8 XCDs (block i -> XCD i%8).
// Give XCD x a contiguous range of tiles so that the workgroups resident on one
// XCD at the same time work on neighbouring tiles of the same (batch, head) and
// share its K/V stream in that XCD's L2.
__device__ __forceinline__ int xcd_tile(int bid, int ntiles) {
  const int q = ntiles >> 3, r = ntiles & 7;
  const int x = bid & 7, slot = bid >> 3;
  return x * q + (x < r ? x : r) + slot;
}

}  // namespace xs
