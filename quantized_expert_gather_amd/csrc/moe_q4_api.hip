// C ABI of the SwitchGLU-q4 MoE library: argument validation, workspace
// layout, path selection and launches.  Every check here runs on the host
// before any GPU work, so invalid calls return a status without touching the
// device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <stdint.h>
#include <string.h>

#include "moe_q4.h"
#include "moe_q4_internal.h"

namespace moeq4 {

static size_t round256(size_t v) { return (v + 255) & ~size_t(255); }

UnionWorkspace union_workspace_layout(int L, int k, int E, int H, int I) {
  (void)E;
  UnionWorkspace w{};
  const size_t pairs = (size_t)L * (size_t)k;
  size_t off = 0;
  w.hdr = off;    off = round256(off + 256);
  w.utab = off;   off = round256(off + pairs * 16);
  w.slot_w = off; off = round256(off + pairs * 4);
  w.slot_dst = off; off = round256(off + pairs * 4);
  w.tcount = off; off = round256(off + (size_t)L * 4);
  w.hbuf = off;   off = round256(off + pairs * (size_t)I * 4);
  w.ys = off;     off = round256(off + pairs * (size_t)H * 4);
  w.ys_dummy = off; off = round256(off + (size_t)H * 4);
  w.total = off;
  return w;
}

__global__ void k_clear_status(uint32_t* hdr) {
  if (threadIdx.x == 0) hdr[0] = 0u;
}

int clear_status_launch(uint32_t* hdr, hipStream_t stream) {
  hipLaunchKernelGGL(k_clear_status, dim3(1), dim3(64), 0, stream, hdr);
  return hipGetLastError() == hipSuccess ? MOE_Q4_OK : MOE_Q4_ERR_LAUNCH;
}

static int shape_status(int L, int k, int E, int H, int I) {
  if (L < 0 || k < 1 || E < 1 || H < 1 || I < 1 || k > E) return MOE_Q4_ERR_SHAPE;
  if (H % 64 || I % 64) return MOE_Q4_ERR_UNSUPPORTED;
  if (E > MOE_Q4_MAX_E) return MOE_Q4_ERR_UNSUPPORTED;
  return MOE_Q4_OK;
}

static int select_path(int L, int k, int E, int H, int I) {
  const int st = shape_status(L, k, E, H, I);
  if (st) return -st;
  if (L == 0) return MOE_Q4_PATH_NONE;
  if (L <= MOE_Q4_UNION_MAX_L && (long)L * k <= MOE_Q4_MAX_PAIRS && union_shape_supported(L, k, E, H, I))
    return MOE_Q4_PATH_UNION;
  if (sorted_shape_supported(L, k, E, H, I)) return MOE_Q4_PATH_SORTED;
  return -MOE_Q4_ERR_UNSUPPORTED;
}

// Codecs other than 4-bit affine group 64 run on the union kernels, with H
// and I multiples of 32 (one scale per 32 inputs at least; 64 for the
// group-64 8-bit affine codes).  More tokens than one union launch serves
// run as consecutive token chunks: at most 32 tokens and 1024 pairs, fewer
// where the chunk's activations would not fit the LDS.  mxfp4 and mxfp8
// inputs longer than that take the sorted (MFMA) path where its streaming
// kernels cover the shape.
static int union_token_cap(int k) { return std::min(MOE_Q4_UNION_MAX_L, MOE_Q4_MAX_PAIRS / k); }

// Tokens per union launch; 0 if not even one token fits.
static int codec_chunk_tokens(int L, int k, int E, int H, int I, int fmt) {
  int c = std::min(L, union_token_cap(k));
  while (c > 0 && !union_shape_supported(c, k, E, H, I, fmt)) --c;
  return c;
}

static bool codec_sorted(int fmt, int L, int k, int E, int H, int I) {
  return (fmt == kFmtMxfp4 || fmt == kFmtMxfp8) && L > union_token_cap(k) && sorted_mx_shape_supported(L, k, E, H, I);
}

static int codec_shape_status(int L, int k, int E, int H, int I, int fmt) {
  if (L < 0 || k < 1 || E < 1 || H < 1 || I < 1 || k > E) return MOE_Q4_ERR_SHAPE;
  const int grp = fmt == kFmtAffine8 ? 64 : 32;
  if (H % grp || I % grp || E > MOE_Q4_MAX_E || k > MOE_Q4_MAX_PAIRS || L > MOE_Q4_CODEC_MAX_L)
    return MOE_Q4_ERR_UNSUPPORTED;
  if (L == 0 || codec_sorted(fmt, L, k, E, H, I)) return MOE_Q4_OK;
  if (codec_chunk_tokens(L, k, E, H, I, fmt) < 1) return MOE_Q4_ERR_UNSUPPORTED;
  return MOE_Q4_OK;
}

// Points the workspace arrays of a sorted-path call into `ws`.
static void sorted_workspace_args(SortedArgs& a, unsigned char* ws, const SortedWorkspace& sw) {
  a.bm = 32 * sorted_row_blocks(a.T, a.k, a.E);
  a.tiles_max = sorted_tiles_max(a.T, a.k, a.E, a.bm);
  a.hdr = reinterpret_cast<uint32_t*>(ws + sw.hdr);
  a.offsets = reinterpret_cast<int32_t*>(ws + sw.offsets);
  a.perm = reinterpret_cast<int32_t*>(ws + sw.perm);
  a.inv = reinterpret_cast<int32_t*>(ws + sw.inv);
  a.rank_tmp = reinterpret_cast<int32_t*>(ws + sw.rank_tmp);
  a.tiles = reinterpret_cast<int4*>(ws + sw.tiles);
  a.asum = reinterpret_cast<float*>(ws + sw.asum);
  a.texp = reinterpret_cast<int32_t*>(ws + sw.texp);
  a.hhi = reinterpret_cast<uint16_t*>(ws + sw.hhi);
  a.hlo = reinterpret_cast<uint16_t*>(ws + sw.hlo);
  a.hsum2 = reinterpret_cast<float*>(ws + sw.hsum2);
  a.ys = reinterpret_cast<float*>(ws + sw.ys);
  a.mxflag_gu = reinterpret_cast<uint32_t*>(ws + sw.mxflag);
  a.mxflag_dn = a.mxflag_gu + sorted_flag_count(a.T, a.k, a.E, a.H, a.I);
}

// Kernel format of a codec; -1 for an unknown codec.
static int codec_fmt(int codec) {
  switch (codec) {
    case MOE_Q4_CODEC_AFFINE4_G64: return kFmtAffine;
    case MOE_Q4_CODEC_AFFINE4_G32: return kFmtAffine32;
    case MOE_Q4_CODEC_MXFP4: return kFmtMxfp4;
    case MOE_Q4_CODEC_NVFP4: return kFmtNvfp4;
    case MOE_Q4_CODEC_AFFINE8_G64: return kFmtAffine8;
    case MOE_Q4_CODEC_MXFP8: return kFmtMxfp8;
  }
  return -1;
}

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

static bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na && nb && x < y + nb && y < x + na;
}

// Compute units of the current device, cached per device (host threads may
// call concurrently: each entry is one atomic int, written once).
static int num_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return -1;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace moeq4

using namespace moeq4;

extern "C" {

size_t moe_swiglu_q4_workspace_bytes(int L, int k, int E, int H, int I) {
  const int path = select_path(L, k, E, H, I);
  if (path <= 0) return 0;
  if (path == MOE_Q4_PATH_SORTED) return sorted_workspace_layout(L, k, E, H, I).total;
  return union_workspace_layout(L, k, E, H, I).total;
}

int moe_swiglu_q4_select_path(int L, int k, int E, int H, int I) { return select_path(L, k, E, H, I); }

int moe_swiglu_q4_forward_stages(const void* x, const int32_t* topk_ids, const float* topk_weights,
                                 const uint32_t* wg, const void* sg, const void* bg, const uint32_t* wu,
                                 const void* su, const void* bu, const uint32_t* wd, const void* sd,
                                 const void* bd, int L, int k, int E, int H, int I, int group_size, int bits,
                                 void* out, int out_dtype, void* workspace, size_t workspace_bytes,
                                 unsigned stages, hipStream_t stream) {
  const int st = shape_status(L, k, E, H, I);
  if (st) return st;
  if (group_size != 64 || bits != 4) return MOE_Q4_ERR_UNSUPPORTED;
  if (out_dtype != MOE_Q4_OUT_BF16 && out_dtype != MOE_Q4_OUT_F32) return MOE_Q4_ERR_UNSUPPORTED;
  if (stages == 0 || (stages & ~MOE_Q4_STAGE_ALL)) return MOE_Q4_ERR_UNSUPPORTED;
  if (L == 0) return MOE_Q4_OK;
  const int path = select_path(L, k, E, H, I);
  if (path < 0) return -path;
  if (!x || !topk_ids || !topk_weights || !wg || !sg || !bg || !wu || !su || !bu || !wd || !sd || !bd || !out)
    return MOE_Q4_ERR_NULL;
  if (!workspace) return MOE_Q4_ERR_WORKSPACE;
  if (!aligned(x, 16) || !aligned(wg, 16) || !aligned(wu, 16) || !aligned(wd, 16) || !aligned(out, 16) ||
      !aligned(topk_ids, 4) || !aligned(topk_weights, 4) || !aligned(sg, 4) || !aligned(bg, 4) ||
      !aligned(su, 4) || !aligned(bu, 4) || !aligned(sd, 4) || !aligned(bd, 4) || !aligned(workspace, 256))
    return MOE_Q4_ERR_ALIGN;
  const size_t ws_need = path == MOE_Q4_PATH_SORTED ? sorted_workspace_layout(L, k, E, H, I).total
                                                     : union_workspace_layout(L, k, E, H, I).total;
  if (workspace_bytes < ws_need) return MOE_Q4_ERR_WORKSPACE;

  const size_t out_bytes = (size_t)L * H * (out_dtype == MOE_Q4_OUT_F32 ? 4 : 2);
  const size_t gu_codes = (size_t)E * I * (H / 8) * 4, gu_sb = (size_t)E * I * (H / 64) * 2;
  const size_t d_codes = (size_t)E * H * (I / 8) * 4, d_sb = (size_t)E * H * (I / 64) * 2;
  const struct { const void* p; size_t n; } ins[] = {
      {x, (size_t)L * H * 2}, {topk_ids, (size_t)L * k * 4}, {topk_weights, (size_t)L * k * 4},
      {wg, gu_codes}, {sg, gu_sb}, {bg, gu_sb}, {wu, gu_codes}, {su, gu_sb}, {bu, gu_sb},
      {wd, d_codes}, {sd, d_sb}, {bd, d_sb}, {workspace, ws_need}};
  for (const auto& in : ins)
    if (overlaps(out, out_bytes, in.p, in.n)) return MOE_Q4_ERR_ALIAS;

  unsigned char* ws = static_cast<unsigned char*>(workspace);
  if (path == MOE_Q4_PATH_SORTED) {
    const SortedWorkspace sw = sorted_workspace_layout(L, k, E, H, I);
    SortedArgs a{};
    a.x = static_cast<const uint16_t*>(x);
    a.ids = topk_ids;
    a.tw = topk_weights;
    a.wg = wg; a.sg = static_cast<const uint16_t*>(sg); a.bg = static_cast<const uint16_t*>(bg);
    a.wu = wu; a.su = static_cast<const uint16_t*>(su); a.bu = static_cast<const uint16_t*>(bu);
    a.wd = wd; a.sd = static_cast<const uint16_t*>(sd); a.bd = static_cast<const uint16_t*>(bd);
    a.out = out;
    a.out_f32 = out_dtype == MOE_Q4_OUT_F32;
    a.T = L; a.k = k; a.E = E; a.H = H; a.I = I;
    a.fmt = kFmtAffine;
    sorted_workspace_args(a, ws, sw);
    return sorted_forward_launch(a, stages, stream);
  }

  const int ncu = num_cus();
  if (ncu <= 0) return MOE_Q4_ERR_LAUNCH;

  const UnionWorkspace lay = union_workspace_layout(L, k, E, H, I);
  UnionArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.ids = topk_ids;
  a.tw = topk_weights;
  a.wg = wg; a.sg = static_cast<const uint16_t*>(sg); a.bg = static_cast<const uint16_t*>(bg);
  a.wu = wu; a.su = static_cast<const uint16_t*>(su); a.bu = static_cast<const uint16_t*>(bu);
  a.wd = wd; a.sd = static_cast<const uint16_t*>(sd); a.bd = static_cast<const uint16_t*>(bd);
  a.out = out;
  a.out_f32 = out_dtype == MOE_Q4_OUT_F32;
  a.L = L; a.k = k; a.E = E; a.H = H; a.I = I;
  // matrix-core tiles for experts with many tokens: whole 4-group iterations
  // over both widths and 8-byte scale pieces
  a.mfma = H % 256 == 0 && I % 256 == 0 && aligned(sg, 8) && aligned(bg, 8) && aligned(su, 8) && aligned(bu, 8) &&
           aligned(sd, 8) && aligned(bd, 8);
  a.hdr = reinterpret_cast<uint32_t*>(ws + lay.hdr);
  a.utab = reinterpret_cast<int4*>(ws + lay.utab);
  a.slot_w = reinterpret_cast<float*>(ws + lay.slot_w);
  a.slot_dst = reinterpret_cast<int32_t*>(ws + lay.slot_dst);
  a.tcount = reinterpret_cast<int32_t*>(ws + lay.tcount);
  a.hbuf = reinterpret_cast<float*>(ws + lay.hbuf);
  a.ys = reinterpret_cast<float*>(ws + lay.ys);
  a.ys_dummy = reinterpret_cast<float*>(ws + lay.ys_dummy);
  return union_forward_launch(a, stages, ncu, stream);
}

int moe_swiglu_q4_forward(const void* x, const int32_t* topk_ids, const float* topk_weights, const uint32_t* wg,
                          const void* sg, const void* bg, const uint32_t* wu, const void* su, const void* bu,
                          const uint32_t* wd, const void* sd, const void* bd, int L, int k, int E, int H, int I,
                          int group_size, int bits, void* out, int out_dtype, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  return moe_swiglu_q4_forward_stages(x, topk_ids, topk_weights, wg, sg, bg, wu, su, bu, wd, sd, bd, L, k, E, H, I,
                                      group_size, bits, out, out_dtype, workspace, workspace_bytes,
                                      MOE_Q4_STAGE_ALL, stream);
}

size_t moe_swiglu_codec_workspace_bytes(int codec, int L, int k, int E, int H, int I) {
  if (codec == MOE_Q4_CODEC_AFFINE4_G64) return moe_swiglu_q4_workspace_bytes(L, k, E, H, I);
  const int fmt = codec_fmt(codec);
  if (fmt < 0 || L == 0 || codec_shape_status(L, k, E, H, I, fmt)) return 0;
  const int Lc = codec_chunk_tokens(L, k, E, H, I, fmt);
  const size_t un = Lc > 0 ? union_workspace_layout(Lc, k, E, H, I).total : 0;
  // enough for the token chunks too, which serve scale arrays not aligned for the sorted path
  return codec_sorted(fmt, L, k, E, H, I) ? std::max(un, sorted_workspace_layout(L, k, E, H, I).total) : un;
}

int moe_swiglu_codec_forward_stages(int codec, const void* x, const int32_t* topk_ids, const float* topk_weights,
                                    const uint32_t* wg, const void* sg, const void* bg, const uint32_t* wu,
                                    const void* su, const void* bu, const uint32_t* wd, const void* sd,
                                    const void* bd, int L, int k, int E, int H, int I, void* out, int out_dtype,
                                    void* workspace, size_t workspace_bytes, unsigned stages, hipStream_t stream) {
  const int fmt = codec_fmt(codec);
  if (fmt < 0) return MOE_Q4_ERR_UNSUPPORTED;
  if (fmt == kFmtAffine)
    return moe_swiglu_q4_forward_stages(x, topk_ids, topk_weights, wg, sg, bg, wu, su, bu, wd, sd, bd, L, k, E, H,
                                        I, 64, 4, out, out_dtype, workspace, workspace_bytes, stages, stream);
  const int st = codec_shape_status(L, k, E, H, I, fmt);
  if (st) return st;
  if (out_dtype != MOE_Q4_OUT_BF16 && out_dtype != MOE_Q4_OUT_F32) return MOE_Q4_ERR_UNSUPPORTED;
  if (stages == 0 || (stages & ~MOE_Q4_STAGE_ALL)) return MOE_Q4_ERR_UNSUPPORTED;
  if (L == 0) return MOE_Q4_OK;
  const int Lc = codec_chunk_tokens(L, k, E, H, I, fmt);
  // the sorted path reads the scale bytes 8 at a time; unaligned ones run as token chunks
  const bool mx_al = aligned(sg, 8) && aligned(su, 8) && aligned(sd, 8);
  const bool srt = codec_sorted(fmt, L, k, E, H, I) && (mx_al || Lc < 1);
  if (srt && !mx_al) return MOE_Q4_ERR_ALIGN;
  // stage-only calls hand the hidden vectors of one launch to the next
  if (!srt && Lc < L && stages != MOE_Q4_STAGE_ALL) return MOE_Q4_ERR_UNSUPPORTED;
  const bool biased = fmt == kFmtAffine32 || fmt == kFmtAffine8;
  if (!x || !topk_ids || !topk_weights || !wg || !sg || !wu || !su || !wd || !sd || !out) return MOE_Q4_ERR_NULL;
  if (biased && (!bg || !bu || !bd)) return MOE_Q4_ERR_NULL;
  if (!workspace) return MOE_Q4_ERR_WORKSPACE;
  // scale (and bias) arrays: bf16 (affine), pairs of E4M3 bytes read as one
  // 16-bit word (nvfp4) or single E8M0 bytes (mxfp4, mxfp8)
  const bool e8m0 = fmt == kFmtMxfp4 || fmt == kFmtMxfp8;
  const size_t sa = e8m0 ? 1 : 2;
  if (!aligned(x, 16) || !aligned(wg, 16) || !aligned(wu, 16) || !aligned(wd, 16) || !aligned(out, 16) ||
      !aligned(topk_ids, 4) || !aligned(topk_weights, 4) || !aligned(workspace, 256) || !aligned(sg, sa) ||
      !aligned(su, sa) || !aligned(sd, sa) || (biased && (!aligned(bg, 2) || !aligned(bu, 2) || !aligned(bd, 2))))
    return MOE_Q4_ERR_ALIGN;
  const UnionWorkspace lay = union_workspace_layout(srt ? 1 : Lc, k, E, H, I);
  const size_t ws_need = srt ? sorted_workspace_layout(L, k, E, H, I).total : lay.total;
  if (workspace_bytes < ws_need) return MOE_Q4_ERR_WORKSPACE;

  // bytes of one scale array per 32 inputs of a row: a bf16 per 32 (affine
  // group 32) or per 64 (8-bit affine), two E4M3 (nvfp4), one E8M0 (mx)
  const size_t per32 = e8m0 || fmt == kFmtAffine8 ? 1 : 2;
  const size_t cb = fmt_8bit(fmt) ? 1 : 2;  // inputs per code byte: 1 (8-bit) or 2 (4-bit)
  const size_t out_bytes = (size_t)L * H * (out_dtype == MOE_Q4_OUT_F32 ? 4 : 2);
  const size_t gu_codes = (size_t)E * I * H / cb, gu_s = (size_t)E * I * (H / 32) * per32;
  const size_t d_codes = (size_t)E * H * I / cb, d_s = (size_t)E * H * (I / 32) * per32;
  const struct { const void* p; size_t n; } ins[] = {
      {x, (size_t)L * H * 2}, {topk_ids, (size_t)L * k * 4}, {topk_weights, (size_t)L * k * 4},
      {wg, gu_codes}, {sg, gu_s}, {wu, gu_codes}, {su, gu_s}, {wd, d_codes}, {sd, d_s},
      {biased ? bg : nullptr, biased ? gu_s : 0}, {biased ? bu : nullptr, biased ? gu_s : 0},
      {biased ? bd : nullptr, biased ? d_s : 0}, {workspace, ws_need}};
  for (const auto& in : ins)
    if (in.p && overlaps(out, out_bytes, in.p, in.n)) return MOE_Q4_ERR_ALIAS;

  if (srt) {
    SortedArgs a{};
    a.x = static_cast<const uint16_t*>(x);
    a.ids = topk_ids;
    a.tw = topk_weights;
    // E8M0 bytes travel in the scale slots; no biases
    a.wg = wg; a.sg = static_cast<const uint16_t*>(sg);
    a.wu = wu; a.su = static_cast<const uint16_t*>(su);
    a.wd = wd; a.sd = static_cast<const uint16_t*>(sd);
    a.out = out;
    a.out_f32 = out_dtype == MOE_Q4_OUT_F32;
    a.T = L; a.k = k; a.E = E; a.H = H; a.I = I;
    a.fmt = fmt;
    sorted_workspace_args(a, static_cast<unsigned char*>(workspace), sorted_workspace_layout(L, k, E, H, I));
    return sorted_forward_launch(a, stages, stream);
  }

  const int ncu = num_cus();
  if (ncu <= 0) return MOE_Q4_ERR_LAUNCH;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  UnionArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.ids = topk_ids;
  a.tw = topk_weights;
  // FP4 formats: the scale bytes travel in the scale slots, the bias slots stay NULL
  a.wg = wg; a.sg = static_cast<const uint16_t*>(sg); a.bg = biased ? static_cast<const uint16_t*>(bg) : nullptr;
  a.wu = wu; a.su = static_cast<const uint16_t*>(su); a.bu = biased ? static_cast<const uint16_t*>(bu) : nullptr;
  a.wd = wd; a.sd = static_cast<const uint16_t*>(sd); a.bd = biased ? static_cast<const uint16_t*>(bd) : nullptr;
  a.fmt = fmt;
  a.out = out;
  a.out_f32 = out_dtype == MOE_Q4_OUT_F32;
  a.L = L; a.k = k; a.E = E; a.H = H; a.I = I;
  a.hdr = reinterpret_cast<uint32_t*>(ws + lay.hdr);
  a.utab = reinterpret_cast<int4*>(ws + lay.utab);
  a.slot_w = reinterpret_cast<float*>(ws + lay.slot_w);
  a.slot_dst = reinterpret_cast<int32_t*>(ws + lay.slot_dst);
  a.tcount = reinterpret_cast<int32_t*>(ws + lay.tcount);
  a.hbuf = reinterpret_cast<float*>(ws + lay.hbuf);
  a.ys = reinterpret_cast<float*>(ws + lay.ys);
  a.ys_dummy = reinterpret_cast<float*>(ws + lay.ys_dummy);
  // token chunks of Lc, in order, on the same workspace
  const size_t out_elt = out_dtype == MOE_Q4_OUT_F32 ? 4 : 2;
  for (int t0 = 0; t0 < L; t0 += Lc) {
    UnionArgs c = a;
    c.L = std::min(Lc, L - t0);
    c.x = a.x + (size_t)t0 * H;
    c.ids = topk_ids + (size_t)t0 * k;
    c.tw = topk_weights + (size_t)t0 * k;
    c.out = static_cast<unsigned char*>(out) + (size_t)t0 * H * out_elt;
    c.status_or = t0 > 0;
    const int st2 = union_forward_launch(c, stages, ncu, stream);
    if (st2) return st2;
  }
  return MOE_Q4_OK;
}

int moe_swiglu_codec_forward(int codec, const void* x, const int32_t* topk_ids, const float* topk_weights,
                             const uint32_t* wg, const void* sg, const void* bg, const uint32_t* wu, const void* su,
                             const void* bu, const uint32_t* wd, const void* sd, const void* bd, int L, int k, int E,
                             int H, int I, void* out, int out_dtype, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  return moe_swiglu_codec_forward_stages(codec, x, topk_ids, topk_weights, wg, sg, bg, wu, su, bu, wd, sd, bd, L, k,
                                         E, H, I, out, out_dtype, workspace, workspace_bytes, MOE_Q4_STAGE_ALL,
                                         stream);
}

size_t moe_swiglu_mxfp4_workspace_bytes(int L, int k, int E, int H, int I) {
  return moe_swiglu_codec_workspace_bytes(MOE_Q4_CODEC_MXFP4, L, k, E, H, I);
}

int moe_swiglu_mxfp4_forward_stages(const void* x, const int32_t* topk_ids, const float* topk_weights,
                                    const uint32_t* wg, const uint8_t* sg, const uint32_t* wu, const uint8_t* su,
                                    const uint32_t* wd, const uint8_t* sd, int L, int k, int E, int H, int I,
                                    void* out, int out_dtype, void* workspace, size_t workspace_bytes,
                                    unsigned stages, hipStream_t stream) {
  return moe_swiglu_codec_forward_stages(MOE_Q4_CODEC_MXFP4, x, topk_ids, topk_weights, wg, sg, nullptr, wu, su,
                                         nullptr, wd, sd, nullptr, L, k, E, H, I, out, out_dtype, workspace,
                                         workspace_bytes, stages, stream);
}

int moe_swiglu_mxfp4_forward(const void* x, const int32_t* topk_ids, const float* topk_weights, const uint32_t* wg,
                             const uint8_t* sg, const uint32_t* wu, const uint8_t* su, const uint32_t* wd,
                             const uint8_t* sd, int L, int k, int E, int H, int I, void* out, int out_dtype,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return moe_swiglu_mxfp4_forward_stages(x, topk_ids, topk_weights, wg, sg, wu, su, wd, sd, L, k, E, H, I, out,
                                         out_dtype, workspace, workspace_bytes, MOE_Q4_STAGE_ALL, stream);
}

int moe_route_union(const int32_t* topk_ids, const float* topk_weights, int L, int k, int E, int32_t* u,
                    int32_t* uniq_ids, uint32_t* tok_mask, float* uniq_w, int32_t* slot_to_uniq,
                    hipStream_t stream) {
  if (L < 1 || k < 1 || E < 1 || k > E) return MOE_Q4_ERR_SHAPE;
  if (L > MOE_Q4_UNION_MAX_L || (long)L * k > MOE_Q4_MAX_PAIRS || E > MOE_Q4_MAX_E) return MOE_Q4_ERR_UNSUPPORTED;
  if (!topk_ids || !topk_weights || !u || !uniq_ids || !tok_mask || !uniq_w || !slot_to_uniq)
    return MOE_Q4_ERR_NULL;
  if (!aligned(topk_ids, 4) || !aligned(topk_weights, 4) || !aligned(u, 4) || !aligned(uniq_ids, 4) ||
      !aligned(tok_mask, 4) || !aligned(uniq_w, 4) || !aligned(slot_to_uniq, 4))
    return MOE_Q4_ERR_ALIGN;
  return route_union_launch(topk_ids, topk_weights, L, k, E, u, uniq_ids, tok_mask, uniq_w, slot_to_uniq, stream);
}

int moe_sort_pairs_tiles_max(int L, int k, int E, int bm) {
  if (L < 0 || k < 1 || E < 1 || bm < 1) return -MOE_Q4_ERR_SHAPE;
  return sorted_tiles_max(L, k, E, bm);
}

int moe_sort_pairs(const int32_t* topk_ids, int L, int k, int E, int bm, int32_t* offsets, int32_t* perm,
                   int32_t* inv, int32_t* tiles, int tiles_cap, uint32_t* info, int32_t* scratch,
                   hipStream_t stream) {
  if (L < 1 || k < 1 || E < 1 || k > E || bm < 1) return MOE_Q4_ERR_SHAPE;
  if (E > MOE_Q4_MAX_E || (long)L * k >= (1L << 30)) return MOE_Q4_ERR_UNSUPPORTED;
  if (!topk_ids || !offsets || !perm || !inv || !tiles || !info || !scratch) return MOE_Q4_ERR_NULL;
  if (tiles_cap < sorted_tiles_max(L, k, E, bm)) return MOE_Q4_ERR_WORKSPACE;
  if (!aligned(topk_ids, 4) || !aligned(offsets, 4) || !aligned(perm, 4) || !aligned(inv, 4) ||
      !aligned(tiles, 16) || !aligned(info, 4) || !aligned(scratch, 4))
    return MOE_Q4_ERR_ALIGN;
  SortedArgs a{};
  a.ids = topk_ids;
  a.T = L; a.k = k; a.E = E;
  a.bm = bm;
  a.tiles_max = tiles_cap;
  a.hdr = info;
  a.offsets = offsets;
  a.perm = perm;
  a.inv = inv;
  a.rank_tmp = scratch;
  a.tiles = reinterpret_cast<int4*>(tiles);
  return sort_launch(a, stream);
}

int moe_q4_read_device_status(const void* workspace, uint32_t* status, uint32_t* last_path, hipStream_t stream) {
  if (!workspace || !status) return MOE_Q4_ERR_NULL;
  if (!aligned(workspace, 256)) return MOE_Q4_ERR_ALIGN;
  uint32_t hdr[4] = {0, 0, 0, 0};
  if (hipStreamSynchronize(stream) != hipSuccess) return MOE_Q4_ERR_LAUNCH;
  if (hipMemcpy(hdr, workspace, sizeof hdr, hipMemcpyDeviceToHost) != hipSuccess) return MOE_Q4_ERR_LAUNCH;
  *status = hdr[0];
  if (last_path) *last_path = hdr[1];
  return MOE_Q4_OK;
}

int moe_q4_clear_device_status(void* workspace, hipStream_t stream) {
  if (!workspace) return MOE_Q4_ERR_NULL;
  if (!aligned(workspace, 256)) return MOE_Q4_ERR_ALIGN;
  return clear_status_launch(static_cast<uint32_t*>(workspace), stream);
}

const char* moe_q4_status_string(int status) {
  switch (status) {
    case MOE_Q4_OK: return "ok";
    case MOE_Q4_ERR_NULL: return "a required pointer is NULL";
    case MOE_Q4_ERR_SHAPE: return "invalid shape (L < 0, k < 1, E < 1, k > E, H or I < 1)";
    case MOE_Q4_ERR_UNSUPPORTED:
      return "unsupported configuration (H or I not a multiple of 64, bits != 4, group != 64, unknown dtype, "
             "or beyond the library limits)";
    case MOE_Q4_ERR_ALIGN: return "pointer misaligned";
    case MOE_Q4_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_Q4_ERR_LAUNCH: return "HIP launch or runtime call failed";
    case MOE_Q4_ERR_ALIAS: return "output overlaps an input or the workspace";
    case MOE_Q4_ERR_SCRATCH:
      return "the shape needs more workspace than the allocation-free entry point's scratch "
             "(MOE_Q4_NOALLOC_SCRATCH_BYTES) holds";
  }
  return "unknown status";
}

}  // extern "C"
