// xs_attn_api.cpp -- the C ABI declared in include/xs_attn.h: argument
// validation (before any HIP call), dispatch to the kernel launchers.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "attn_launch.h"
#include "xs_attn.h"

// Device memory of xs_attn_fwd_noalloc: the split-key partials of one call
// (fp32 partial O, then per-row running max and row sum), the same contents a
// caller workspace holds.  Every GPU the library runs on holds its own copy
// from the time the library's code is loaded onto it until the process ends.
// Host code never passes `scratch` itself (in host code the name is only a
// stand-in): it uses the per-device address from hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[XS_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kVersion = 1 * 10000 + 5 * 100 + 0;
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
  // K/V rows of one (batch, head) are addressed with 32-bit buffer offsets
  if ((double)S * H * D * (double)in_elem_bytes >= 4294967296.0) return XS_ERR_UNSUPPORTED;
  // query tiles (and the half-height tiles of a second launch) are counted in
  // 32-bit integers
  if ((double)B * H * ((S + xs::kHalfM - 1) / xs::kHalfM) > 2147483647.0) return XS_ERR_UNSUPPORTED;
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
  args->groups = 0;
  args->npair = 0;
  args->dp = 0;
  args->units = 0;
  args->ws_o = nullptr;
  args->ws_ml = nullptr;
  args->batch_rows = S;
  args->chunk_rows = 0;
  args->jump_rows = 0;
  args->lse = nullptr;
  args->half = 0;
  args->tile0 = 0;
  return XS_OK;
}

// Input layout and the optional log-sum-exp output, on validated arguments.
int apply_layout_and_lse(xs::AttnArgs* a, int in_layout, float* lse, size_t in_elem_bytes) {
  if (in_layout != XS_LAYOUT_BSHD && in_layout != XS_LAYOUT_CHUNKED) return XS_ERR_UNSUPPORTED;
  // With B = 1 or P = 1 the chunk layout is byte-identical to [B][S][H][D].
  if (in_layout == XS_LAYOUT_CHUNKED && a->B > 1 && a->P > 1) {
    if (a->T % xs::kBlockN != 0) return XS_ERR_UNSUPPORTED;  // K/V blocks may not straddle chunks
    a->batch_rows = a->T;
    a->chunk_rows = a->T;
    a->jump_rows = (long long)(a->B - 1) * a->T;
  }
  if (lse) {
    if (((uintptr_t)lse & 3u) != 0) return XS_ERR_ALIGN;
    const size_t n = (size_t)a->B * a->S * a->H * a->D;
    const size_t lse_bytes = (size_t)a->B * a->H * a->S * sizeof(float);
    const size_t in_bytes = n * in_elem_bytes;
    if (overlaps(lse, lse_bytes, a->q, in_bytes) || overlaps(lse, lse_bytes, a->k, in_bytes) ||
        overlaps(lse, lse_bytes, a->v, in_bytes) || overlaps(lse, lse_bytes, a->out, n * 2))
      return XS_ERR_OVERLAP;
    a->lse = lse;
  }
  return XS_OK;
}

int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    return 256;
  return n;
}

// Work schedule (attn_launch.h, Sched): `groups` workgroups; each takes dp
// whole tiles in rounds, then an equal share of the remaining tiles' units
// (query tile, pair of key blocks), cutting a tile wherever a share ends inside
// it (partials + merge).  Candidates: groups = tiles (one whole tile each),
// groups = k * tiles (k = 2 .. 16: every tile in k equal pieces, one round) and
// groups = the resident slots (one persistent workgroup per CU: dp = tiles /
// slots rounds of whole tiles, then the remainder shared).  The plan picks the
// cheapest by a run-time model: rounds of resident workgroups x (units per
// workgroup + 1.5 units of prologue/epilogue per piece) x time per unit, plus,
// when tiles are cut, the partials' HBM traffic and the merge launch; cutting
// must gain 3 % over the best uncut schedule.  Calls whose best schedule cuts
// nothing run the tiles left after the whole rounds (at most half a round of
// them) as half-height tiles in a second launch, one per slot: a round of
// twice as many half tiles instead of a last round that leaves half of the
// chip or more idle.
struct Plan {
  int groups, npair, dp;
  long long units, tiles;  // units of the remainder tiles
  bool cut;
  // second launch: half tiles [half0, half0 + halves) (none when halves = 0;
  // groups = 0 when there are no whole rounds before it)
  long long half0 = 0;
  int halves = 0;
};

// Invariant kept for the kernels and the merge: units == 0 or units >= groups
// (every share owns at least one remainder unit).
Plan make_plan(long long groups, int npair, long long tiles) {
  long long dp = groups <= tiles ? tiles / groups : 0;
  while (dp > 0 && tiles > dp * groups && (tiles - dp * groups) * npair < groups) --dp;
  const long long units = (tiles - dp * groups) * npair;
  // every remainder share boundary floor(c*units/groups) must be a multiple of npair
  const bool cut = units > 0 && !(units % groups == 0 && (units / groups) % npair == 0);
  return Plan{(int)groups, npair, (int)dp, units, tiles, cut};
}

double plan_cost(const Plan& p, int slots, int D) {
  const double t_pair = 2.0 * (D == 128 ? 1.9e-6 : 1.0e-6);  // s per 2 key blocks per workgroup
  const double hbm = 4.0e12, t_launch = 5.0e-6, ovh = 1.5;
  const double rounds = (double)((p.groups + slots - 1) / slots);
  const long long per = (p.units + p.groups - 1) / p.groups;  // remainder units per share
  double pieces;  // most remainder pieces in one share
  if (per == 0)
    pieces = 0.0;
  else if (!p.cut)
    pieces = (double)(per / p.npair);
  else if (p.units % p.groups == 0 && p.npair % per == 0)
    pieces = 1.0;  // shares of equal size that tile each tile exactly
  else
    pieces = (double)((per + p.npair - 1) / p.npair) + 1.0;
  double t = rounds * ((double)p.dp * (p.npair + ovh) + (double)per + ovh * pieces) * t_pair;
  if (p.cut) {
    // at most one cut tile per share boundary, each in about groups/tiles + 1 pieces
    const double rtiles = (double)p.units / p.npair;
    const double cut_tiles = (double)p.groups < rtiles ? (double)p.groups : rtiles;
    const double ratio = (double)p.groups / rtiles + 1.0;
    const double pieces_per_tile = ratio > 2.0 ? ratio : 2.0;
    t += cut_tiles * xs::kBlockM * (pieces_per_tile * (4.0 * D + 8.0) + 2.0 * D) / hbm + t_launch;
  }
  return t;
}

// The half-tile form of an uncut schedule (halves = 0 when it has none): dp
// whole rounds of full tiles on every slot, then the remaining tiles as half
// tiles, when those fit one round.
Plan with_half_tiles(int B, int S, int H, int npair, int slots) {
  const long long mt = (S + xs::kBlockM - 1) / xs::kBlockM, mh = (S + xs::kHalfM - 1) / xs::kHalfM;
  const long long tiles = (long long)B * H * mt;
  const long long dp = tiles / slots, t0 = dp * slots;
  Plan p = dp > 0 ? make_plan(slots, npair, t0) : Plan{0, npair, 0, 0, 0, false};
  if (t0 == tiles) return p;
  const long long bh0 = t0 / mt;
  p.half0 = bh0 * mh + 2 * (t0 - bh0 * mt);
  const long long halves = (long long)B * H * mh - p.half0;
  if (halves > slots) p.halves = 0;
  else p.halves = (int)halves;
  return p;
}

// True when `p` is device memory of the current device.  A kernel completes
// only when its stores are visible where they went, so with out_packed behind
// a link (host memory, a peer GPU) a second launch would first wait for the
// whole last round of the first to drain instead of overlapping that drain with
// the next tiles' computation; half tiles are used only for local outputs.
bool local_device_memory(const void* p) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  const hipError_t before = hipPeekAtLastError();
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    // a pointer the runtime does not know: take the one-launch schedule and
    // leave no error of this query behind (an earlier one stays reported)
    if (before == hipSuccess) (void)hipGetLastError();
    return false;
  }
  return at.type == hipMemoryTypeDevice && at.device == dev;
}

Plan plan_for(int B, int S, int H, int D, bool allow_cut, bool half_ok = false) {
  const long long tiles = (long long)B * H * ((S + xs::kBlockM - 1) / xs::kBlockM);
  const int nblk = (S + xs::kBlockN - 1) / xs::kBlockN;
  const int npair = (nblk + 1) / 2;
  const int slots = device_cus() * xs::kGroupsPerCU;
  Plan best = make_plan(tiles, npair, tiles);
  double best_cost = plan_cost(best, slots, D);
  auto consider = [&](long long g) {
    if (g < 1 || g > tiles * npair || g > 0x7fffffffLL) return;
    const Plan p = make_plan(g, npair, tiles);
    if (p.cut && !allow_cut) return;
    const double c = plan_cost(p, slots, D);
    if ((p.cut && c < 0.97 * best_cost) || (!p.cut && c <= best_cost)) {
      best = p;
      best_cost = c;
    }
  };
  consider(slots);  // persistent: one workgroup per slot
  for (int k = 2; k <= 16 && k <= npair; ++k)
    if (tiles * k <= slots) consider(tiles * k);  // k equal pieces per tile, one round
  if (half_ok && !best.cut && tiles % slots != 0) {
    const Plan h = with_half_tiles(B, S, H, npair, slots);
    if (h.halves > 0) return h;
  }
  return best;
}

size_t workspace_bytes(const Plan& pl, int D) {
  if (!pl.cut) return 0;
  return 2 * (size_t)pl.groups * xs::kBlockM * ((size_t)D * 4 + 8);
}

// Attaches the schedule and, when it cuts tiles, the workspace to validated
// arguments (inputs of in_elem_bytes per element).  Without a workspace the
// schedule never cuts.
int attach_workspace(xs::AttnArgs* a, void* ws, size_t ws_bytes, size_t in_elem_bytes,
                     Plan* plan, bool one_launch = false) {
  if (ws != nullptr && ((uintptr_t)ws & 15u) != 0) return XS_ERR_ALIGN;
  Plan pl = plan_for(a->B, a->S, a->H, a->D, ws != nullptr, !one_launch);
  if (pl.halves > 0 && !local_device_memory(a->out))
    pl = plan_for(a->B, a->S, a->H, a->D, ws != nullptr, false);
  *plan = pl;
  const size_t need = workspace_bytes(pl, a->D);
  if (need > 0 && ws_bytes < need) return XS_ERR_WORKSPACE;
  if (need > 0) {
    // the partials must not land in an input or an output
    const size_t n = (size_t)a->B * a->S * a->H * a->D;
    const size_t in_bytes = n * in_elem_bytes;
    if (overlaps(ws, need, a->q, in_bytes) || overlaps(ws, need, a->k, in_bytes) ||
        overlaps(ws, need, a->v, in_bytes) || overlaps(ws, need, a->out, n * 2) ||
        (a->lse && overlaps(ws, need, a->lse, (size_t)a->B * a->H * a->S * sizeof(float))))
      return XS_ERR_OVERLAP;
  }
  a->groups = pl.groups;
  a->npair = pl.npair;
  a->dp = pl.dp;
  a->units = pl.units;
  if (need > 0) {
    a->ws_o = (float*)ws;
    a->ws_ml = (float*)((char*)ws + 2 * (size_t)pl.groups * xs::kBlockM * a->D * 4);
  }
  return XS_OK;
}

// Device address of `scratch` on the current device, looked up once per device
// (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return XS_ERR_LAUNCH;
  if (dev >= kMaxDevices) return XS_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return XS_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return XS_OK;
}

int launch(const xs::AttnArgs& a, const Plan& pl, bool fp8, hipStream_t stream) {
  if (a.groups > 0) {
    const hipError_t e = fp8 ? xs::launch_attn_fp8(a, stream) : xs::launch_attn_bf16(a, stream);
    if (e != hipSuccess) return XS_ERR_LAUNCH;
  }
  if (pl.halves > 0) {
    xs::AttnArgs h = a;
    h.half = 1;
    h.tile0 = (int)pl.half0;
    h.groups = pl.halves;
    h.dp = 1;
    h.units = 0;
    h.ws_o = nullptr;
    h.ws_ml = nullptr;
    const hipError_t e = fp8 ? xs::launch_attn_fp8(h, stream) : xs::launch_attn_bf16(h, stream);
    if (e != hipSuccess) return XS_ERR_LAUNCH;
  }
  if (a.ws_o != nullptr && xs::launch_attn_combine(a, stream) != hipSuccess) return XS_ERR_LAUNCH;
  return XS_OK;
}

}  // namespace

extern "C" {

int xs_attn_fwd_ex(const void* q, const void* k, const void* v, int in_layout, void* out_packed,
                   float* lse, int B, int S, int H_local, int D, int P, float scale,
                   void* workspace, size_t workspace_bytes, void* stream) {
  xs::AttnArgs a;
  int rc = validate(q, k, v, out_packed, B, S, H_local, D, P, scale, 2, &a);
  if (rc != XS_OK) return rc;
  const bool one_launch = (in_layout & XS_ONE_LAUNCH) != 0;
  rc = apply_layout_and_lse(&a, in_layout & ~XS_ONE_LAUNCH, lse, 2);
  if (rc != XS_OK) return rc;
  Plan pl;
  rc = attach_workspace(&a, workspace, workspace_bytes, 2, &pl, one_launch);
  if (rc != XS_OK) return rc;
  return launch(a, pl, false, (hipStream_t)stream);
}

int xs_attn_fwd_ws(const void* q, const void* k, const void* v, void* out_packed, int B, int S,
                   int H_local, int D, int P, float scale, void* workspace, size_t workspace_bytes,
                   void* stream) {
  return xs_attn_fwd_ex(q, k, v, XS_LAYOUT_BSHD, out_packed, nullptr, B, S, H_local, D, P, scale,
                        workspace, workspace_bytes, stream);
}

int xs_attn_fwd(const void* q, const void* k, const void* v, void* out_packed, int B, int S,
                int H_local, int D, int P, float scale, void* stream) {
  return xs_attn_fwd_ex(q, k, v, XS_LAYOUT_BSHD, out_packed, nullptr, B, S, H_local, D, P, scale,
                        nullptr, 0, stream);
}

int xs_attn_fwd_fp8_ex(const void* q8, const void* k8, const void* v8, int in_layout,
                       float q_descale, float k_descale, float v_descale, void* out_packed,
                       float* lse, int B, int S, int H_local, int D, int P, float scale,
                       void* workspace, size_t workspace_bytes, void* stream) {
  xs::AttnArgs a;
  int rc = validate(q8, k8, v8, out_packed, B, S, H_local, D, P, scale, 1, &a);
  if (rc != XS_OK) return rc;
  const bool one_launch = (in_layout & XS_ONE_LAUNCH) != 0;
  rc = apply_layout_and_lse(&a, in_layout & ~XS_ONE_LAUNCH, lse, 1);
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
  Plan pl;
  rc = attach_workspace(&a, workspace, workspace_bytes, 1, &pl, one_launch);
  if (rc != XS_OK) return rc;
  return launch(a, pl, true, (hipStream_t)stream);
}

int xs_attn_fwd_fp8_ws(const void* q8, const void* k8, const void* v8, float q_descale,
                       float k_descale, float v_descale, void* out_packed, int B, int S,
                       int H_local, int D, int P, float scale, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return xs_attn_fwd_fp8_ex(q8, k8, v8, XS_LAYOUT_BSHD, q_descale, k_descale, v_descale,
                            out_packed, nullptr, B, S, H_local, D, P, scale, workspace,
                            workspace_bytes, stream);
}

int xs_attn_fwd_fp8(const void* q8, const void* k8, const void* v8, float q_descale,
                    float k_descale, float v_descale, void* out_packed, int B, int S, int H_local,
                    int D, int P, float scale, void* stream) {
  return xs_attn_fwd_fp8_ex(q8, k8, v8, XS_LAYOUT_BSHD, q_descale, k_descale, v_descale,
                            out_packed, nullptr, B, S, H_local, D, P, scale, nullptr, 0, stream);
}

int xs_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out_packed, int B,
                        int S, int H_local, int D, int P, float scale, void* stream) {
  xs::AttnArgs a;
  int rc = validate(q, k, v, out_packed, B, S, H_local, D, P, scale, 2, &a);
  if (rc != XS_OK) return rc;
  const size_t need = workspace_bytes(plan_for(B, S, H_local, D, true), D);
  if (need > (size_t)XS_NOALLOC_SCRATCH_BYTES) return XS_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    rc = scratch_address(&ws);
    if (rc != XS_OK) return rc;
  }
  Plan pl;
  rc = attach_workspace(&a, ws, (size_t)XS_NOALLOC_SCRATCH_BYTES, 2, &pl);
  if (rc != XS_OK) return rc;
  return launch(a, pl, false, (hipStream_t)stream);
}

size_t xs_attn_workspace_size(int B, int S, int H_local, int D) {
  if (B < 1 || S < 1 || H_local < 1 || (D != 64 && D != 128)) return 0;
  return workspace_bytes(plan_for(B, S, H_local, D, true), D);
}

int xs_attn_schedule_ex(int B, int S, int H_local, int D, int with_workspace, int fp8,
                        int* groups, int* whole_rounds, int* pieces, int* half_tiles) {
  if (B < 1 || S < 1 || H_local < 1 || (D != 64 && D != 128)) return XS_ERR_SHAPE;
  (void)fp8;  // bf16 and fp8 calls run the same schedule
  const Plan p = plan_for(B, S, H_local, D, with_workspace != 0, true);
  if (groups) *groups = p.groups;
  if (whole_rounds) *whole_rounds = p.dp;
  if (half_tiles) *half_tiles = p.halves;
  if (pieces) {
    int most = 1;
    if (p.cut) {
      const xs::Sched sch{p.units, p.groups, p.npair, p.dp};
      for (long long t = 0; t < p.units / p.npair; ++t) {  // remainder tiles
        const int n = sch.owner((t + 1) * p.npair - 1) - sch.owner(t * p.npair) + 1;
        most = n > most ? n : most;
      }
    }
    *pieces = most;
  }
  return XS_OK;
}

int xs_attn_schedule(int B, int S, int H_local, int D, int with_workspace, int* groups,
                     int* whole_rounds, int* pieces) {
  return xs_attn_schedule_ex(B, S, H_local, D, with_workspace, 0, groups, whole_rounds, pieces,
                             nullptr);
}

int xs_attn_split_count(int B, int S, int H_local, int D) {
  if (B < 1 || S < 1 || H_local < 1 || (D != 64 && D != 128)) return 0;
  const Plan p = plan_for(B, S, H_local, D, true);
  if (!p.cut) return 1;
  const xs::Sched sch{p.units, p.groups, p.npair, p.dp};
  int most = 1;
  for (long long t = 0; t < p.units / p.npair; ++t) {  // remainder tiles
    const int n = sch.owner((t + 1) * p.npair - 1) - sch.owner(t * p.npair) + 1;
    most = n > most ? n : most;
  }
  return most;
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
      return "unsupported argument: D must be 64 or 128, scales finite, the input layout known "
             "(chunked inputs with B > 1 and P > 1 need S/P to be a multiple of 64)";
    case XS_ERR_ALIGN:
      return "a pointer is not 16-byte aligned";
    case XS_ERR_LAUNCH:
      return "the HIP kernel launch failed";
    case XS_ERR_OVERLAP:
      return "buffers overlap: out_packed, lse or the workspace shares memory with another buffer";
    case XS_ERR_WORKSPACE:
      return "workspace smaller than xs_attn_workspace_size()";
    case XS_ERR_SCRATCH:
      return "xs_attn_fwd_noalloc: the shape's split-key partials need more than the library's "
             "static scratch of XS_NOALLOC_SCRATCH_BYTES bytes (use xs_attn_fwd_ws)";
    default:
      return "unknown status code";
  }
}

int xs_attn_version(void) { return kVersion; }

}  // extern "C"
