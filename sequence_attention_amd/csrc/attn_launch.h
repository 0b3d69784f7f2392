// attn_launch.h -- host-side launchers of the attention kernels (internal to
// the library; the public interface is include/xs_attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xs {

struct AttnArgs {
  const void* q;  // [B][S][H][D], bf16 or e4m3
  const void* k;
  const void* v;
  void* out;      // bf16 [P][B][T][H][D]
  int B, S, H, D, P, T;
  float c;        // |scale| * log2(e), times q_descale * k_descale for fp8
  int neg;        // nonzero when scale < 0: queries are negated as they are loaded
  float o_scale;  // factor applied with 1/l in the epilogue (v_descale for fp8)
  // Split of the key range: work item (b, h, split, m-tile) covers key blocks
  // [split*nb_per, min(nblk, (split+1)*nb_per)).  With nsplit > 1 the items
  // write unnormalised fp32 partials (O, and m, l per row) to the workspace
  // and attn_combine merges them into out.
  int nsplit;
  int nb_per;
  float* ws_o;    // [nsplit][B*H*S][D] fp32
  float* ws_ml;   // [nsplit][B*H*S][2] fp32: running max (log2 units), row sum
  // Input layout.  Row s of batch b of an input tensor starts at row index
  //   b*batch_rows + s + (chunk_rows ? s / chunk_rows : 0) * jump_rows
  // (in units of H*D elements): [B][S][H][D] has batch_rows = S, chunk_rows =
  // 0; the chunk layout [P][B][T][H][D] has batch_rows = T, chunk_rows = T,
  // jump_rows = (B-1)*T.
  int batch_rows;
  int chunk_rows;
  long long jump_rows;
  float* lse;     // NULL or [B][H][S] fp32 log-sum-exp (natural log)
};

// Tile geometry shared by the bf16 and fp8 kernels and the host-side plan.
#ifndef XS_BM
#define XS_BM 256
#endif
#ifndef XS_WGPC
#define XS_WGPC 1
#endif
constexpr int kBlockM = XS_BM;         // query rows per workgroup
constexpr int kBlockN = 64;            // keys per K/V block
constexpr int kGroupsPerCU = XS_WGPC;  // workgroups resident per compute unit

hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t stream);

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t stream);
hipError_t launch_attn_fp8(const AttnArgs& a, hipStream_t stream);

}  // namespace xs
