// Host/device interface between the C ABI and the union-path kernels.  Internal header.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moeq4 {

// Weight formats of the union kernels (a template parameter of each kernel).
constexpr int kFmtAffine = 0;    // 4-bit affine, bf16 scale and bias per 64 inputs
constexpr int kFmtMxfp4 = 1;     // FP4 E2M1, E8M0 scale per 32 inputs
constexpr int kFmtNvfp4 = 2;     // FP4 E2M1, FP8 E4M3 scale per 16 inputs
constexpr int kFmtAffine32 = 3;  // 4-bit affine, bf16 scale and bias per 32 inputs
constexpr int kFmtAffine8 = 4;   // 8-bit affine, bf16 scale and bias per 64 inputs
constexpr int kFmtMxfp8 = 5;     // FP8 E4M3, E8M0 scale per 32 inputs
// FP4 element formats: converted in hardware into natural-order pairs, no bias
__host__ __device__ constexpr bool fmt_fp4(int f) { return f == kFmtMxfp4 || f == kFmtNvfp4; }
__host__ __device__ constexpr bool fmt_8bit(int f) { return f == kFmtAffine8 || f == kFmtMxfp8; }
// staged activations / hidden vectors in natural element order (else the
// 4-bit affine nibble-pair order)
__host__ __device__ constexpr bool fmt_natural(int f) { return fmt_fp4(f) || fmt_8bit(f); }
// a per-group bias (affine) and so per-position activation sums
__host__ __device__ constexpr bool fmt_biased(int f) { return !fmt_fp4(f) && f != kFmtMxfp8; }
// 16-byte loads per position of the activations; a position is the inputs of
// one 16-byte weight load: 32 for 4-bit codes, 16 for 8-bit codes
__host__ __device__ constexpr int fmt_na(int f) { return fmt_8bit(f) ? 2 : 4; }
__host__ __device__ constexpr int fmt_pos_inputs(int f) { return 8 * fmt_na(f); }
// LDS stride of one token's staged activations (one pair slot's hidden
// vector) in 16-byte units, for a width of `inputs`: 2 bytes an input plus
// one pad unit, so the rows of a matrix-core operand (one token each) fall
// in different LDS banks
__host__ __device__ constexpr int lds_row_units(int inputs) { return inputs / 8 + 1; }

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
  // workspace regions (pairs = L * k is an upper bound on (expert, token) pairs)
  uint32_t* hdr;    // [0] status of the last call, [1] its path, [2] its distinct experts u
  int4* utab;       // [u] (expert id, token mask, first pair slot, 0) per distinct expert
  float* slot_w;    // [pairs] router weight of each (expert, token) pair
  int32_t* slot_dst;  // [pairs] output row of each pair slot in ys: t * k + c, c = rank of its expert among t's
  int32_t* tcount;  // [L] number of pair slots of each token
  float* hbuf;      // [pairs][I] hidden vectors h = silu(gate) * up, fp32
  float* ys;        // [L * k][H] router-weighted down outputs, token-major (row t * k + c)
  float* ys_dummy;  // [H] write sink for token slots past an expert's count
  // dynamic LDS layout of the gate/up kernel
  size_t lds_act, lds_asum, lds_union;
  int dn_slots;  // pair slots the down kernel stages in LDS at a time
  int dn_rows;   // one token: down blocks own output rows of all experts and write out (no combine kernel)
  int status_or; // later token chunk of one call: OR this chunk's status into the call's status word
  int fmt;       // weight format (kFmt*): for the FP4 formats sg/su/sd hold scale bytes, bg/bu/bd unused
  int mfma;      // 4-bit affine banks that the matrix-core tiles can read (widths multiples of 256, scale
                 // arrays 8-byte aligned): experts with many tokens take them
  size_t lds_mlist;  // gate/up LDS: the distinct experts on the matrix cores, then the others ([2][pairs])
  size_t lds_red;    // gate/up LDS: the waves' partial tile sums ([kWaves][8][64] fp32)
};

// Workspace layout (byte offsets from the workspace base, 256-aligned regions).
struct UnionWorkspace {
  size_t hdr, utab, slot_w, slot_dst, tcount, hbuf, ys, ys_dummy, total;
};

UnionWorkspace union_workspace_layout(int L, int k, int E, int H, int I);
bool union_shape_supported(int L, int k, int E, int H, int I, int fmt = kFmtAffine);
size_t union_lds_bytes_max(int L, int k, int E, int H, int I, int fmt = kFmtAffine);
int union_forward_launch(const UnionArgs& a, unsigned stages, int num_cu, hipStream_t stream);
int route_union_launch(const int32_t* ids, const float* tw, int L, int k, int E, int32_t* u, int32_t* uniq_ids,
                       uint32_t* tok_mask, float* uniq_w, int32_t* slot_to_uniq, hipStream_t stream);
int clear_status_launch(uint32_t* hdr, hipStream_t stream);

// Arguments of one sorted-path forward (T tokens, P = T * k pairs).
struct SortedArgs {
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
  int T, k, E, H, I;
  int fmt;            // kFmtAffine, or kFmtMxfp4 / kFmtMxfp8 (scale slots hold E8M0 bytes, no biases)
  int bm;             // rows per tile (32, 64 or 128)
  int tiles_max;      // capacity of `tiles`
  uint32_t* hdr;      // [0] status, [1] path, [2] valid pairs, [3] tiles
  int32_t* offsets;   // [E+1] first sorted row of each expert; [E] = valid pairs
  int32_t* perm;      // [P] sorted row -> pair (valid pairs by (expert, pair), then invalid ones)
  int32_t* inv;       // [P] pair -> sorted row
  int32_t* rank_tmp;  // [P] pairs scattered into their expert's segment, unordered
  int4* tiles;        // [tiles_max] (expert, first sorted row, rows, 0)
  float* asum;        // [T][H/64] per-token sums of x over each 64-input group
  int32_t* texp;      // [T] exponent of each token's largest |x| (frexp; 0 for x = 0)
  uint16_t* hhi;      // [P][I] bf16 hi of h, columns in code order inside each 8
  uint16_t* hlo;      // [P][I] bf16 lo of h (h - hi, rounded)
  float* hsum2;       // [P][I/32] sum of hi + lo over each 32 columns
  float* ys;          // [P][H] per-pair down outputs, unweighted
  uint32_t* mxflag_gu;  // mxfp4: per gate/up block, 1 if it needs the exact pass
  uint32_t* mxflag_dn;  // mxfp4: per down block, likewise
};

struct SortedWorkspace {
  size_t hdr, offsets, perm, inv, rank_tmp, tiles, asum, texp, hhi, hlo, hsum2, ys, mxflag, total;
};

int sorted_row_blocks(int T, int k, int E);
int sorted_tiles_max(int T, int k, int E, int bm);
size_t sorted_flag_count(int T, int k, int E, int H, int I);
SortedWorkspace sorted_workspace_layout(int T, int k, int E, int H, int I);
bool sorted_shape_supported(int T, int k, int E, int H, int I);
// mxfp4 and mxfp8 banks on the sorted path: the streaming kernels, H and I multiples of 256
bool sorted_mx_shape_supported(int T, int k, int E, int H, int I);
int sort_launch(const SortedArgs& a, hipStream_t stream);
int sorted_forward_launch(const SortedArgs& a, unsigned stages, hipStream_t stream);

}  // namespace moeq4
