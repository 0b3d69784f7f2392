// xs_attn_api.cpp -- the C ABI declared in include/xs_attn.h: argument
// validation (before any HIP call), dispatch to the kernel launchers.
#include <math.h>
#include <stdint.h>

#include "attn_launch.h"
#include "xs_attn.h"

namespace {

constexpr int kVersion = 1 * 10000 + 0 * 100 + 0;
constexpr float kLog2e = 1.4426950408889634f;

// |scale| * log2(e): the kernels compute p = 2^(s*c - m).  A zero scale is
// replaced by a factor so small that s*c rounds every exponent to 0 (p = 1,
// the uniform softmax) while masked scores (-inf) still give p = 0 instead of
// the NaN of -inf * 0.
float scores_factor(float scale) {
  const float c = fabsf(scale) * kLog2e;
  return c > 1e-30f ? c : 1e-30f;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

// Shared validation of both entry points; fills `args` on success.
int validate(const void* q, const void* k, const void* v, void* out, int B, int S, int H, int D,
             int P, float scale, size_t in_elem_bytes, xs::AttnArgs* args) {
  if (!q || !k || !v || !out) return XS_ERR_NULL;
  if (B < 1 || S < 1 || H < 1 || D < 1 || P < 1) return XS_ERR_SHAPE;
  if (S % P != 0) return XS_ERR_SHAPE;
  if (D != 64 && D != 128) return XS_ERR_UNSUPPORTED;
  if (!isfinite(scale)) return XS_ERR_UNSUPPORTED;
  // element counts must fit comfortably in 64-bit byte offsets
  const double elems = (double)B * (double)S * (double)H * (double)D;
  if (elems * 2.0 > 9.0e18) return XS_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return XS_ERR_ALIGN;
  const size_t n = (size_t)B * S * H * D;
  const size_t in_bytes = n * in_elem_bytes, out_bytes = n * 2;
  if (overlaps(out, out_bytes, q, in_bytes) || overlaps(out, out_bytes, k, in_bytes) ||
      overlaps(out, out_bytes, v, in_bytes))
    return XS_ERR_OVERLAP;
  args->q = q;
  args->k = k;
  args->v = v;
  args->out = out;
  args->B = B;
  args->S = S;
  args->H = H;
  args->D = D;
  args->P = P;
  args->T = S / P;
  args->neg = scale < 0.0f;
  args->c = scores_factor(scale);
  args->o_scale = 1.0f;
  return XS_OK;
}

}  // namespace

extern "C" {

int xs_attn_fwd(const void* q, const void* k, const void* v, void* out_packed, int B, int S,
                int H_local, int D, int P, float scale, void* stream) {
  xs::AttnArgs a;
  int rc = validate(q, k, v, out_packed, B, S, H_local, D, P, scale, 2, &a);
  if (rc != XS_OK) return rc;
  if (xs::launch_attn_bf16(a, (hipStream_t)stream) != hipSuccess) return XS_ERR_LAUNCH;
  return XS_OK;
}

int xs_attn_fwd_fp8(const void* q8, const void* k8, const void* v8, float q_descale,
                    float k_descale, float v_descale, void* out_packed, int B, int S, int H_local,
                    int D, int P, float scale, void* stream) {
  xs::AttnArgs a;
  int rc = validate(q8, k8, v8, out_packed, B, S, H_local, D, P, scale, 1, &a);
  if (rc != XS_OK) return rc;
  if (!isfinite(q_descale) || !isfinite(k_descale) || !isfinite(v_descale))
    return XS_ERR_UNSUPPORTED;
  // softmax(scale * (q8 dq)(k8 dk)) = softmax(scale*dq*dk * q8.k8); V's descale
  // commutes with the normalised weighted sum and is applied in the epilogue.
  const float qk = scale * q_descale * k_descale;
  if (!isfinite(qk)) return XS_ERR_UNSUPPORTED;
  a.neg = qk < 0.0f;
  a.c = scores_factor(qk);
  a.o_scale = v_descale;
  if (xs::launch_attn_fp8(a, (hipStream_t)stream) != hipSuccess) return XS_ERR_LAUNCH;
  return XS_OK;
}

const char* xs_attn_strerror(int status) {
  switch (status) {
    case XS_OK:
      return "success";
    case XS_ERR_NULL:
      return "a required pointer is NULL";
    case XS_ERR_SHAPE:
      return "invalid shape: B, S, H_local, D and P must be >= 1 and S a multiple of P";
    case XS_ERR_UNSUPPORTED:
      return "unsupported argument: D must be 64 or 128 and scales finite";
    case XS_ERR_ALIGN:
      return "a pointer is not 16-byte aligned";
    case XS_ERR_LAUNCH:
      return "the HIP kernel launch failed";
    case XS_ERR_OVERLAP:
      return "out_packed overlaps q, k or v";
    default:
      return "unknown status code";
  }
}

int xs_attn_version(void) { return kVersion; }

}  // extern "C"
