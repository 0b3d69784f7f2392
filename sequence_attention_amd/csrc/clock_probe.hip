// clock_probe.hip -- xs_clock_stamp (include/xs_probe.h): per-workgroup samples
// of the shader clock counter and the constant-rate counter, for the average
// shader clock over the work between two stamps on one stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "xs_probe.h"

namespace xs {

__global__ __launch_bounds__(64) void clock_stamp_kernel(unsigned long long* stamp) {
  const unsigned long long t = __builtin_amdgcn_s_memtime();
  const unsigned long long r = __builtin_amdgcn_s_memrealtime();
  // hardware register 20 (XCC_ID), bits 3:0: the XCD this wave runs on
  const unsigned xcc = __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 0xFu;
  if (threadIdx.x == 0) {
    unsigned long long* s = stamp + 4 * blockIdx.x;
    s[0] = t;
    s[1] = r;
    s[2] = xcc;
    s[3] = 0;
  }
}

}  // namespace xs

extern "C" int xs_clock_stamp(void* stamp, int* wall_khz, void* stream) {
  if (stamp == nullptr) return -1;
  if (((uintptr_t)stamp & 7u) != 0) return -4;
  if (wall_khz != nullptr) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(wall_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
      return -5;
  }
  hipLaunchKernelGGL(xs::clock_stamp_kernel, dim3(XS_CLOCK_STAMP_WORDS / 4), dim3(64), 0,
                     (hipStream_t)stream, (unsigned long long*)stamp);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
