// Host/device interface between the C ABI and the union-path kernels.  Internal header.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moeq4 {

// Arguments of one union-path forward (device pointers; LDS offsets in bytes).
struct UnionArgs {
  const uint16_t* x;
  const int32_t* ids;
  const float* tw;
  const uint32_t* wg;
  const uint16_t* sg;
  const uint16_t* bg;
  const uint32_t* wu;
  const uint16_t* su;
  const uint16_t* bu;
  const uint32_t* wd;
  const uint16_t* sd;
  const uint16_t* bd;
  void* out;
  int out_f32;
  int L, k, E, H, I;
  // workspace regions
  uint32_t* hdr;    // [0] status of the last call, [1] its path, [2] its distinct experts
  uint32_t* cnt;    // [H/32] per-row-block arrival counters of the down kernel
  uint32_t* hbuf;   // [pairs][I/32][32] hidden vectors as bf16 hi/lo pairs
  float* hsum;      // [pairs][I/32] per-32-row sums of hi + lo
  float* ys;        // [pairs][H] router-weighted down outputs per (expert, token)
  // dynamic LDS layout
  size_t lds_act, lds_asum, lds_hpair, lds_hval, lds_toks, lds_tokw, lds_flag, lds_union;
};

// Workspace layout (byte offsets from the workspace base, 256-aligned regions).
struct UnionWorkspace {
  size_t hdr, cnt, hbuf, hsum, ys, total;
};

UnionWorkspace union_workspace_layout(int L, int k, int E, int H, int I);
bool union_shape_supported(int L, int k, int E, int H, int I);
size_t union_lds_bytes_max(int L, int k, int E, int H, int I);
int union_forward_launch(const UnionArgs& a, unsigned stages, int num_cu, hipStream_t stream);
int route_union_launch(const int32_t* ids, const float* tw, int L, int k, int E, int32_t* u, int32_t* uniq_ids,
                       uint32_t* tok_mask, float* uniq_w, int32_t* slot_to_uniq, hipStream_t stream);
int clear_status_launch(uint32_t* hdr, hipStream_t stream);

}  // namespace moeq4
