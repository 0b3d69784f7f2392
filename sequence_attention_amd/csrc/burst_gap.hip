// burst_gap.hip -- the Burst-Gap microbenchmark: producers issue bursts of
// stores into a destination (fine-grained host memory standing in for a remote
// link), separated by a computation-free gap, and time how long each burst takes
// to issue.
//
// Model being characterised (X-Stage paper, gist.science explainer, "Methodik:
// Die X-Stage-Abstraktion und das Burst-Gap-Modell"): the sender-visible issue
// time of a burst of aggregate volume V from K producers that leave a gap G
// between bursts is T_iss(G; K, V) = max(T0_iss(K, V), V/R - G), with T0_iss
// the backpressure-free issue time, R the effective drain rate and Q the
// outstanding capacity (volume in flight before the issue stalls).  On one GPU
// the "remote stores" are ordinary vector stores to host-coherent memory over
// PCIe: issued stores retire into the memory pipeline and drain while the wave
// moves on, until the pipeline's outstanding capacity is exhausted.
//
// Each producer is one workgroup of 4 waves; lane i of a burst step stores 16
// bytes at offset 16*(step*256 + i) of the producer's region, so a burst is a
// fully coalesced sweep of `bytes` bytes.  Successive bursts go to successive
// regions of a ring that the destination holds.  Every wave records, per burst, the
// shader clocks from its first store to the issue of its last store (no wait
// for completion), then spins `gap_cycles` clocks without memory traffic.
// After the last burst it records how long its stores take to complete.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "device_common.h"
#include "xs_burst_gap.h"

namespace xs {

struct BurstGapArgs {
  uint8_t* dst;
  unsigned long long* times;
  size_t bytes;          // per producer and burst
  long long gap_cycles;
  int nburst;
  int producers;
  int ring;              // regions of producers*bytes bytes in dst, used in turn
};

constexpr int kBgThreads = 256;
constexpr int kBgWaves = kBgThreads / 64;

__global__ __launch_bounds__(kBgThreads) void burst_gap_kernel(BurstGapArgs a) {
  const int p = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const size_t steps = a.bytes / (16 * kBgThreads);
  const int stride = a.nburst + 3;
  unsigned long long* out = a.times + ((size_t)p * kBgWaves + wave) * stride;

  __builtin_amdgcn_s_barrier();
  const uint64_t c_start = __builtin_amdgcn_s_memtime();
  const uint64_t r_start = __builtin_amdgcn_s_memrealtime();
  for (int b = 0; b < a.nburst; ++b) {
    const u32x4 val = {(uint32_t)p, (uint32_t)threadIdx.x, (uint32_t)b, 0x5eedu};
    // burst b fills region b % ring, so bursts write fresh addresses while the
    // ring lasts (as output tiles do), not lines still held in a cache
    uint8_t* region = a.dst + ((size_t)(b % a.ring) * a.producers + p) * a.bytes;
    asm volatile("" ::: "memory");
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    for (size_t s = 0; s < steps; ++s)
      *(u32x4*)(region + 16 * (s * kBgThreads + threadIdx.x)) = val;
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    asm volatile("" ::: "memory");
    if (lane == 0) out[b] = t1 - t0;
    // the gap: computation-free spin on the clock (no memory traffic)
    const uint64_t g_end = t1 + (uint64_t)a.gap_cycles;
    while (__builtin_amdgcn_s_memtime() < g_end) __builtin_amdgcn_s_sleep(1);
  }
  const uint64_t d0 = __builtin_amdgcn_s_memtime();
  wait_vmcnt<0>();
  const uint64_t d1 = __builtin_amdgcn_s_memtime();
  const uint64_t r_end = __builtin_amdgcn_s_memrealtime();
  if (lane == 0) {
    out[a.nburst] = d1 - d0;                // drain of the last burst after its gap
    out[a.nburst + 1] = d1 - c_start;       // shader clocks of the whole walk
    out[a.nburst + 2] = r_end - r_start;    // 100 MHz ticks of the whole walk
  }
}

// The same measurement with the attention epilogue's own store pattern: a
// producer is a workgroup of 8 waves that owns one 256-row output tile; wave w
// stores rows 32w .. 32w+31, each row_bytes long and row_pitch bytes apart (the
// rows of one head in the destination-ordered buffer are H*D*2 bytes apart), as
// row_bytes/16 store instructions of 8 bytes per lane -- lane l writes bytes
// 16c + 8(l/32) .. +7 of row l%32 in instruction c, i.e. 16 bytes into each of
// 32 rows per instruction, exactly as the attention kernels' epilogue does.
// With `coupled`, each wave waits for its burst's stores to complete (s_waitcnt
// vmcnt(0)) before the gap and the recorded time is that completion time: the
// attention kernels do the same implicitly, since the wait for the next tile's
// K/V loads before its first barrier also waits for the stores issued before
// it (loads and stores share the vector-memory counter).
struct BurstTileArgs {
  uint8_t* dst;
  unsigned long long* times;
  long long gap_cycles;
  int row_bytes;
  int row_pitch;
  int nburst;
  int producers;
  int ring;     // regions of producers * 256 * row_pitch bytes in dst, used in turn
  int coupled;  // wait for the burst's stores to complete before the gap
  const uint8_t* gap_src;  // gap of loads: device memory of gap_mask + 1 bytes (or NULL)
  size_t gap_mask;
  int gap_loads;           // 1 KiB per wave each, issued together, then waited for
};

constexpr int kTileRows = 256;
constexpr int kTileThreads = 512;
constexpr int kTileWaves = kTileThreads / 64;

__global__ __launch_bounds__(kTileThreads) void burst_tile_kernel(BurstTileArgs a) {
  const int p = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = wave * 32 + (lane & 31);
  const int chunks = a.row_bytes / 16;
  const int stride = 2 * a.nburst + 3;
  unsigned long long* out = a.times + ((size_t)p * kTileWaves + wave) * stride;
  const size_t region_bytes = (size_t)kTileRows * a.row_pitch;
  u32x4 acc = {0u, 0u, 0u, 0u};

  __builtin_amdgcn_s_barrier();
  const uint64_t c_start = __builtin_amdgcn_s_memtime();
  const uint64_t r_start = __builtin_amdgcn_s_memrealtime();
  for (int b = 0; b < a.nburst; ++b) {
    const u32x2 val = {(uint32_t)p, (uint32_t)b};
    uint8_t* rowp = a.dst + ((size_t)(b % a.ring) * a.producers + p) * region_bytes +
                    (size_t)row * a.row_pitch + 8 * (lane >> 5);
    asm volatile("" ::: "memory");
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    for (int c = 0; c < chunks; ++c) *(u32x2*)(rowp + 16 * c) = val;
    if (a.coupled) wait_vmcnt<0>();  // as a wave that waits on its memory counter next
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    asm volatile("" ::: "memory");
    if (lane == 0) out[b] = t1 - t0;
    if (a.gap_src != nullptr) {
      // the gap as a tile's key loop sees it: loads from device memory (fresh
      // addresses every burst), issued together and waited for
      const size_t base = (((size_t)b * a.producers + p) * kTileWaves + wave) * a.gap_loads;
      for (int i = 0; i < a.gap_loads; ++i)
        acc ^= *(const u32x4*)(a.gap_src + ((((base + i) << 10) + 16 * lane) & a.gap_mask));
      keep(acc);
      const uint64_t t2 = __builtin_amdgcn_s_memtime();
      if (lane == 0) out[a.nburst + b] = t2 - t1;
    } else {
      const uint64_t g_end = t1 + (uint64_t)a.gap_cycles;
      while (__builtin_amdgcn_s_memtime() < g_end) __builtin_amdgcn_s_sleep(1);
      if (lane == 0) out[a.nburst + b] = __builtin_amdgcn_s_memtime() - t1;
    }
  }
  const uint64_t d0 = __builtin_amdgcn_s_memtime();
  wait_vmcnt<0>();
  const uint64_t d1 = __builtin_amdgcn_s_memtime();
  const uint64_t r_end = __builtin_amdgcn_s_memrealtime();
  if (lane == 0) {
    out[2 * a.nburst] = d1 - d0;
    out[2 * a.nburst + 1] = d1 - c_start;
    out[2 * a.nburst + 2] = r_end - r_start;
  }
}

}  // namespace xs

extern "C" int xs_burst_gap_tiles(void* dst, size_t dst_bytes, int producers, int row_bytes,
                                  int row_pitch, int nburst, long long gap_cycles, int coupled,
                                  const void* gap_src, size_t gap_src_bytes, int gap_loads,
                                  unsigned long long* times, void* stream) {
  if (!dst || !times) return XS_BG_ERR_NULL;
  if (gap_src != nullptr &&
      (gap_loads < 1 || gap_loads > 65536 || gap_src_bytes < 4096 ||
       (gap_src_bytes & (gap_src_bytes - 1)) != 0))
    return XS_BG_ERR_ARG;
  if (gap_src != nullptr && ((uintptr_t)gap_src & 15u) != 0) return XS_BG_ERR_ALIGN;
  if (producers < 1 || producers > 4096 || nburst < 1 || nburst > 4096 || gap_cycles < 0 ||
      gap_cycles > (1LL << 32) || (long long)nburst * gap_cycles > (1LL << 34) ||
      row_bytes < 16 || row_bytes > 4096 || row_bytes % 16 != 0 || row_pitch < row_bytes ||
      row_pitch % 16 != 0 || row_pitch > (1 << 20))
    return XS_BG_ERR_ARG;
  if (((uintptr_t)dst & 15u) != 0 || ((uintptr_t)times & 7u) != 0) return XS_BG_ERR_ALIGN;
  const size_t per_burst = (size_t)producers * xs::kTileRows * (size_t)row_pitch;
  if (dst_bytes < per_burst) return XS_BG_ERR_ARG;
  const size_t ring = dst_bytes / per_burst;
  xs::BurstTileArgs a{(uint8_t*)dst, times, gap_cycles, row_bytes, row_pitch, nburst, producers,
                      (int)(ring < (size_t)nburst ? ring : (size_t)nburst), coupled != 0,
                      (const uint8_t*)gap_src, gap_src_bytes - 1, gap_loads};
  void* kargs[] = {&a};
  if (hipLaunchKernel((const void*)xs::burst_tile_kernel, dim3((unsigned)producers),
                      dim3(xs::kTileThreads), kargs, 0, (hipStream_t)stream) != hipSuccess)
    return XS_BG_ERR_LAUNCH;
  return 0;
}

extern "C" int xs_burst_gap(void* dst, size_t dst_bytes, int producers, size_t bytes, int nburst,
                            long long gap_cycles, unsigned long long* times, void* stream) {
  if (!dst || !times) return XS_BG_ERR_NULL;
  if (producers < 1 || producers > 4096 || nburst < 1 || nburst > 4096 || gap_cycles < 0 ||
      gap_cycles > (1LL << 32) || (long long)nburst * gap_cycles > (1LL << 34) || bytes == 0 ||
      bytes % (16 * xs::kBgThreads) != 0 || bytes > ((size_t)1 << 30))
    return XS_BG_ERR_ARG;
  if (((uintptr_t)dst & 15u) != 0 || ((uintptr_t)times & 7u) != 0) return XS_BG_ERR_ALIGN;
  const size_t per_burst = (size_t)producers * bytes;
  if (dst_bytes < per_burst) return XS_BG_ERR_ARG;
  const size_t ring = dst_bytes / per_burst;
  xs::BurstGapArgs a{(uint8_t*)dst, times, bytes, gap_cycles, nburst, producers,
                     (int)(ring < (size_t)nburst ? ring : (size_t)nburst)};
  void* kargs[] = {&a};
  if (hipLaunchKernel((const void*)xs::burst_gap_kernel, dim3((unsigned)producers),
                      dim3(xs::kBgThreads), kargs, 0, (hipStream_t)stream) != hipSuccess)
    return XS_BG_ERR_LAUNCH;
  return 0;
}
