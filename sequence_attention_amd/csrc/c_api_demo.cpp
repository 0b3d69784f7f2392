// c_api_demo.cpp -- uses the library through its C ABI alone: no Python, no
// torch.  Device buffers come from the HIP runtime; the call is xs_attn_fwd on
// a small share.  Every key of a (batch, head) carries the same value row, so
// each output row must equal that row exactly (the softmax weights of a row
// sum to one and the row's values are exact in bf16): this checks the batch,
// head and dimension placement of the destination-ordered output without a
// reference implementation.  Invalid calls must return the documented status
// codes.  Exit status 0 on success.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "xs_attn.h"

namespace {

uint16_t bf16_bits(float f) {  // round to nearest even
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

float bf16_value(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// the value row of (b, h): k/8 for k < 256 has at most 8 significant bits
float value_of(int b, int h, int d, int H) { return (float)(((b * H + h) * 64 + d) % 256) / 8.0f; }

bool hip_ok(hipError_t e, const char* what) {
  if (e == hipSuccess) return true;
  std::fprintf(stderr, "c_api_demo: %s failed: %s\n", what, hipGetErrorString(e));
  return false;
}

}  // namespace

int main() {
  const int B = 2, S = 384, H = 3, D = 64, P = 4, T = S / P;
  const size_t n = (size_t)B * S * H * D;
  std::vector<uint16_t> q(n), k(n), v(n), out(n);
  uint32_t state = 12345u;  // 32-bit LCG for the queries and keys
  auto next = [&]() {
    state = state * 1664525u + 1013904223u;
    return (float)(state >> 8) / 16777216.0f * 4.0f - 2.0f;  // [-2, 2)
  };
  for (int b = 0; b < B; ++b)
    for (int s = 0; s < S; ++s)
      for (int h = 0; h < H; ++h)
        for (int d = 0; d < D; ++d) {
          const size_t i = (((size_t)b * S + s) * H + h) * D + d;
          q[i] = bf16_bits(next());
          k[i] = bf16_bits(next());
          v[i] = bf16_bits(value_of(b, h, d, H));
        }

  void *dq = nullptr, *dk = nullptr, *dv = nullptr, *dout = nullptr;
  const size_t bytes = n * sizeof(uint16_t);
  if (!hip_ok(hipMalloc(&dq, bytes), "hipMalloc") || !hip_ok(hipMalloc(&dk, bytes), "hipMalloc") ||
      !hip_ok(hipMalloc(&dv, bytes), "hipMalloc") || !hip_ok(hipMalloc(&dout, bytes), "hipMalloc"))
    return 1;
  if (!hip_ok(hipMemcpy(dq, q.data(), bytes, hipMemcpyHostToDevice), "hipMemcpy") ||
      !hip_ok(hipMemcpy(dk, k.data(), bytes, hipMemcpyHostToDevice), "hipMemcpy") ||
      !hip_ok(hipMemcpy(dv, v.data(), bytes, hipMemcpyHostToDevice), "hipMemcpy"))
    return 1;

  const float scale = 1.0f / std::sqrt((float)D);
  int rc = xs_attn_fwd(dq, dk, dv, dout, B, S, H, D, P, scale, nullptr);
  if (rc != XS_OK) {
    std::fprintf(stderr, "c_api_demo: xs_attn_fwd returned %d (%s)\n", rc, xs_attn_strerror(rc));
    return 1;
  }
  if (!hip_ok(hipDeviceSynchronize(), "kernel") ||
      !hip_ok(hipMemcpy(out.data(), dout, bytes, hipMemcpyDeviceToHost), "hipMemcpy"))
    return 1;
  // out_packed[p][b][s'][h][d] = O[b][p*T + s'][h][d] = value_of(b, h, d)
  size_t bad = 0;
  for (int p = 0; p < P; ++p)
    for (int b = 0; b < B; ++b)
      for (int sp = 0; sp < T; ++sp)
        for (int h = 0; h < H; ++h)
          for (int d = 0; d < D; ++d) {
            const size_t i = ((((size_t)p * B + b) * T + sp) * H + h) * D + d;
            if (bf16_value(out[i]) != value_of(b, h, d, H)) ++bad;
          }
  if (bad) {
    std::fprintf(stderr, "c_api_demo: %zu of %zu output elements differ from their value row\n", bad, n);
    return 1;
  }

  // documented status codes of invalid calls (validated before any HIP call)
  struct Case {
    const char* what;
    int got, want;
  } cases[] = {
      {"S not a multiple of P", xs_attn_fwd(dq, dk, dv, dout, B, S, H, D, 5, scale, nullptr), XS_ERR_SHAPE},
      {"null q", xs_attn_fwd(nullptr, dk, dv, dout, B, S, H, D, P, scale, nullptr), XS_ERR_NULL},
      {"D = 96", xs_attn_fwd(dq, dk, dv, dout, B, S, H, 96, P, scale, nullptr), XS_ERR_UNSUPPORTED},
      {"scale not finite", xs_attn_fwd(dq, dk, dv, dout, B, S, H, D, P, NAN, nullptr), XS_ERR_UNSUPPORTED},
      {"out_packed overlapping q", xs_attn_fwd(dq, dk, dv, dq, B, S, H, D, P, scale, nullptr), XS_ERR_OVERLAP},
  };
  for (const Case& c : cases)
    if (c.got != c.want) {
      std::fprintf(stderr, "c_api_demo: %s returned %d (%s), expected %d\n", c.what, c.got,
                   xs_attn_strerror(c.got), c.want);
      return 1;
    }

  hipFree(dq);
  hipFree(dk);
  hipFree(dv);
  hipFree(dout);
  std::printf("c_api_demo: ok (xs_attn version %d, %zu outputs exact, %zu invalid calls rejected)\n",
              xs_attn_version(), n, sizeof(cases) / sizeof(cases[0]));
  return 0;
}
