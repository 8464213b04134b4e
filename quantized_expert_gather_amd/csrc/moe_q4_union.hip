// Union path of the SwitchGLU-q4 MoE layer for gfx950 (MI355X): the exported
// route-union kernel, the combine kernel and the launchers.  The gate/up and
// down kernel templates live in moe_q4_union_kernels.h and are instantiated
// in the moe_q4_inst_*.hip units (compiled in parallel).
#include <algorithm>
#include <mutex>

#include "moe_q4_union_kernels.h"
#include "moe_q4_inst.h"

namespace moeq4 {

// ---------------------------------------------------------------------------
// route union (exported)
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_route_union(const int32_t* __restrict__ ids, const float* __restrict__ tw,
                                                     int L, int k, int E, int32_t* __restrict__ u_out,
                                                     int32_t* __restrict__ uniq_ids, uint32_t* __restrict__ tok_mask,
                                                     float* __restrict__ uniq_w, int32_t* __restrict__ slot_to_uniq,
                                                     int u_max) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int P = L * k;
  UnionLds s;
  carve_union(smem, E, P, s);
  stage_routes(ids, tw, P, s);
  build_union(P, k, E, s);
  const int u = s.scal[0];
  const int tid = threadIdx.x;
  if (tid == 0) *u_out = u;
  for (int i = tid; i < u_max; i += blockDim.x) {
    uniq_ids[i] = i < u ? s.uniq[i] : -1;
    tok_mask[i] = i < u ? s.mask[i] : 0u;
  }
  for (int it = tid; it < u_max * L; it += blockDim.x) {
    const int i = it / L, t = it % L;
    float v = 0.0f;
    if (i < u && ((s.mask[i] >> t) & 1u)) v = token_expert_weight(s, t, k, s.uniq[i]);
    uniq_w[it] = v;
  }
  for (int p = tid; p < P; p += blockDim.x) {
    const int e = ids[p];
    int r = -1;
    if (e >= 0 && e < E) r = s.scan[e >> 5] + __popc(s.bitmap[e >> 5] & ((1u << (e & 31)) - 1u));
    slot_to_uniq[p] = r;
  }
}

// ---------------------------------------------------------------------------
// combine: out[t, m] = sum over c < tcount[t] (ascending expert) of ys[t * k + c, m]
// All k rows are loaded at once (rows past the count are ignored), so the
// kernel waits for memory once.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_combine(UnionArgs a) {
  const int H = a.H, k = a.k;
  const int n4 = H >> 2;
  const int it = blockIdx.x * blockDim.x + threadIdx.x;  // one float4 of one token
  const int t = blockIdx.y;
  if (it >= n4) return;
  const int cnt = a.tcount[t];
  const float4* rows = reinterpret_cast<const float4*>(a.ys + (size_t)t * k * H) + it;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  int c = 0;
  for (; c + 8 <= k; c += 8) {
    float4 v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = rows[(size_t)(c + q) * n4];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      // rows past the count hold stale data: select, never add them
      const float4 w = c + q < cnt ? v[q] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      acc.x += w.x; acc.y += w.y; acc.z += w.z; acc.w += w.w;
    }
  }
  for (; c < cnt; ++c) {
    const float4 v = rows[(size_t)c * n4];
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  if (a.out_f32) {
    reinterpret_cast<float4*>(a.out)[(size_t)t * n4 + it] = acc;
  } else {
    const uint32_t lo = f32_to_bf16_rne(acc.x) | (f32_to_bf16_rne(acc.y) << 16);
    const uint32_t hi = f32_to_bf16_rne(acc.z) | (f32_to_bf16_rne(acc.w) << 16);
    reinterpret_cast<uint2*>(a.out)[(size_t)t * n4 + it] = make_uint2(lo, hi);
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

namespace {

int lanes_per_row(int KU) {
  int lpr = 2;
  while (lpr < KU && lpr < 64) lpr <<= 1;
  return lpr;
}

// positions per lane, rounded up to an instantiated count (0: unsupported)
int positions_per_lane(int KU, int lpr, bool down) {
  const int ppl = (KU + lpr - 1) / lpr;
  static const int kGu[] = {1, 2, 3, 4, 6, 8};
  static const int kDn[] = {1, 2, 4};
  if (down) {
    for (int v : kDn)
      if (ppl <= v) return v;
  } else {
    for (int v : kGu)
      if (ppl <= v) return v;
  }
  return 0;
}

size_t align16(size_t v) { return (v + 15) & ~size_t(15); }

size_t union_lds(int E, int P) { return (size_t)4 * (2 * ((E + 31) >> 5) + 5 * P + 1 + 2); }

// gate/up LDS: activations of all L tokens | their 32-input sums | route
// union | the matrix-core expert list | (matrix-core instances) the waves'
// partial tile sums
size_t gateup_lds_layout(UnionArgs& a, bool mf = false) {
  const int KU = a.H / fmt_pos_inputs(a.fmt);  // positions; the activations take 2 H bytes per token
  size_t off = 0;
  a.lds_act = off;   off = align16(off + (size_t)a.L * lds_row_units(a.H) * 16);
  a.lds_asum = off;  off = align16(off + (size_t)a.L * KU * 4);
  a.lds_union = off; off = align16(off + union_lds(a.E, a.L * a.k));
  a.lds_mlist = off; off = align16(off + (size_t)8 * a.L * a.k);
  a.lds_red = off;
  if (mf) off = align16(off + (size_t)kWaves * 8 * 64 * 4);
  return off;
}

// Matrix-core instances run only above this many tokens: at or below it an
// expert rarely gathers enough tokens to pay for the tiles, and the GEMV
// instances keep their own register budget.
constexpr int kMfmaMinL = 8;
bool use_mfma(const UnionArgs& a) { return a.fmt == kFmtAffine && a.mfma && a.L > kMfmaMinL; }

constexpr size_t kMaxLds = 160 * 1024;

struct OccCache {
  const void* fn;
  size_t lds;
  int blocks;
};

// Resident blocks per CU of a kernel at an LDS size, cached (host threads may
// call concurrently, so the cache is guarded).
int blocks_per_cu(const void* fn, int threads, size_t lds) {
  static std::mutex mu;
  static OccCache cache[64];
  static int n = 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    for (int c = 0; c < n; ++c)
      if (cache[c].fn == fn && cache[c].lds == lds) return cache[c].blocks;
  }
  int b = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, fn, threads, lds) != hipSuccess || b < 1) b = 1;
  std::lock_guard<std::mutex> lock(mu);
  if (n < 64) cache[n++] = OccCache{fn, lds, b};
  return b;
}

}  // namespace

size_t union_lds_bytes_max(int L, int k, int E, int H, int I, int fmt) {
  UnionArgs a{};
  a.L = L; a.k = k; a.E = E; a.H = H; a.I = I; a.fmt = fmt;
  return gateup_lds_layout(a);
}

bool union_shape_supported(int L, int k, int E, int H, int I, int fmt) {
  const int pos = fmt_pos_inputs(fmt), KG = H / pos, KD = I / pos;
  const int lg = lanes_per_row(KG), ld = lanes_per_row(KD);
  if (!positions_per_lane(KG, lg, false) || !positions_per_lane(KD, ld, true)) return false;
  if ((I % (gateup_rows(positions_per_lane(KG, lg, false)) * (64 / lg))) != 0) return false;
  // a down step covers whole row steps of every expert
  if (H % ((64 / ld) * down_rows(64 / ld)) != 0) return false;
  return union_lds_bytes_max(L, k, E, H, I, fmt) <= kMaxLds &&
         down_lds_head(L * k) + down_slot_bytes(KD, fmt_na(fmt)) + 256 <= kMaxLds;
}

int route_union_launch(const int32_t* ids, const float* tw, int L, int k, int E, int32_t* u, int32_t* uniq_ids,
                       uint32_t* tok_mask, float* uniq_w, int32_t* slot_to_uniq, hipStream_t stream) {
  const int P = L * k;
  const int u_max = P < E ? P : E;
  hipLaunchKernelGGL(k_route_union, dim3(1), dim3(256), union_lds(E, P), stream, ids, tw, L, k, E, u, uniq_ids,
                     tok_mask, uniq_w, slot_to_uniq, u_max);
  return hipGetLastError() == hipSuccess ? MOE_Q4_OK : MOE_Q4_ERR_LAUNCH;
}

int union_forward_launch(const UnionArgs& base, unsigned stages, int num_cu, hipStream_t stream) {
  const int P = base.L * base.k;
  const int u_max = P < base.E ? P : base.E;
  if (stages & MOE_Q4_STAGE_GATEUP) {
    UnionArgs a = base;
    const int KU = a.H / fmt_pos_inputs(a.fmt);
    const int lpr = lanes_per_row(KU), ppl = positions_per_lane(KU, lpr, false);
    const void* fn = use_mfma(a) && gateup_lds_layout(a, true) <= kMaxLds ? gateup_kernel_mf(lpr, ppl, lpr * ppl == KU)
                                                                           : nullptr;
    const size_t lds = gateup_lds_layout(a, fn != nullptr);
    if (!fn)
      fn = a.fmt != kFmtAffine ? gateup_kernel_fmt(a.fmt, lpr, ppl, lpr * ppl == KU)
                               : gateup_kernel(lpr, ppl, lpr * ppl == KU, (a.H / 64) % 2 == 0);
    if (!fn || lds > kMaxLds) return MOE_Q4_ERR_UNSUPPORTED;
    const int wunits = u_max * (a.I / (gateup_rows(ppl) * (64 / lpr)));
    int grid = num_cu * blocks_per_cu(fn, kThreads, lds);
    const int need = (wunits + kWaves - 1) / kWaves;
    if (grid > need) grid = need;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(reinterpret_cast<void (*)(UnionArgs)>(const_cast<void*>(fn)), dim3(grid), dim3(kThreads),
                       lds, stream, a);
    if (hipGetLastError() != hipSuccess) return MOE_Q4_ERR_LAUNCH;
  }
  if (stages & MOE_Q4_STAGE_DOWN) {
    UnionArgs a = base;
    const int KU = a.I / fmt_pos_inputs(a.fmt), NA = fmt_na(a.fmt);
    const int lpr = lanes_per_row(KU), ppl = positions_per_lane(KU, lpr, true);
    // as many pair slots staged at once as the LDS holds, up to all of them
    const size_t base_lds = down_lds_head(P);
    const size_t slot_bytes = down_slot_bytes(KU, NA);
    if (base_lds + slot_bytes + 256 > kMaxLds) return MOE_Q4_ERR_UNSUPPORTED;
    a.dn_slots = (int)std::min<size_t>((size_t)P, (kMaxLds - 256 - base_lds) / slot_bytes);
    size_t lds = base_lds + (size_t)a.dn_slots * slot_bytes;
    const bool qs = a.fmt == kFmtAffine && (a.I / 64) % 2 == 0;
    // one token per register pass when every expert has exactly one token
    // (L = 1), or when a lane holds several positions per row (a second
    // token's hidden vectors would not fit in the registers beside the ring)
    const int nt = (a.L == 1 || ppl >= 2) ? 1 : 2;
    // one token: each block owns whole output rows of every expert (all pair
    // slots staged at once plus a row slice per slot) and writes out, so the
    // combine kernel is not needed
    const int wstep = (64 / lpr) * down_rows(64 / lpr);
    const int blk_rows = ((a.H / wstep + num_cu - 1) / num_cu) * wstep;
    const size_t rows_lds = base_lds + (size_t)P * slot_bytes + (size_t)P * blk_rows * 4;
    a.dn_rows = a.L == 1 && rows_lds + 256 <= kMaxLds;
    if (a.dn_rows) {
      a.dn_slots = P;
      lds = rows_lds;
    }
    const void* fn = use_mfma(a) && !a.dn_rows && down_threads(nt, ppl) == 512
                         ? down_kernel_mf(lpr, ppl, lpr * ppl == KU, nt)
                         : nullptr;
    if (!fn)
      fn = a.fmt != kFmtAffine ? down_kernel_fmt(a.fmt, lpr, ppl, lpr * ppl == KU, nt)
                               : down_kernel(lpr, ppl, lpr * ppl == KU, qs, nt);
    if (!fn || lds > kMaxLds) return MOE_Q4_ERR_UNSUPPORTED;
    // one block per CU: the CU's waves share the block's converted hidden
    // vectors and its work counter
    hipLaunchKernelGGL(reinterpret_cast<void (*)(UnionArgs)>(const_cast<void*>(fn)), dim3(num_cu),
                       dim3(down_threads(nt, ppl)), lds, stream, a);
    if (hipGetLastError() != hipSuccess) return MOE_Q4_ERR_LAUNCH;
    if (a.dn_rows) return MOE_Q4_OK;
    dim3 cgrid((a.H / 4 + 255) / 256, a.L);
    hipLaunchKernelGGL(k_combine, cgrid, dim3(256), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return MOE_Q4_ERR_LAUNCH;
  }
  return MOE_Q4_OK;
}

}  // namespace moeq4

namespace moeq4 {

const void* gateup_kernel(int lpr, int ppl, bool full, bool qs) {
  const void* f = gateup_kernel_0(lpr, ppl, full, qs);
  if (!f) f = gateup_kernel_1(lpr, ppl, full, qs);
  if (!f) f = gateup_kernel_2(lpr, ppl, full, qs);
  if (!f) f = gateup_kernel_3(lpr, ppl, full, qs);
  return f;
}

const void* down_kernel(int lpr, int ppl, bool full, bool qs, int nt) {
  const void* f = down_kernel_0(lpr, ppl, full, qs, nt);
  if (!f) f = down_kernel_1(lpr, ppl, full, qs, nt);
  if (!f) f = down_kernel_2(lpr, ppl, full, qs, nt);
  if (!f) f = down_kernel_3(lpr, ppl, full, qs, nt);
  return f;
}

const void* gateup_kernel_mf(int lpr, int ppl, bool full) {
  const void* f = gateup_kernel_mf_0(lpr, ppl, full);
  return f ? f : gateup_kernel_mf_1(lpr, ppl, full);
}

const void* down_kernel_mf(int lpr, int ppl, bool full, int nt) { return down_kernel_mf_0(lpr, ppl, full, nt); }

const void* gateup_kernel_fmt(int fmt, int lpr, int ppl, bool full) {
  const void* f = nullptr;
  switch (fmt) {
    case kFmtMxfp4: f = gateup_kernel_mxfp4_0(lpr, ppl, full); return f ? f : gateup_kernel_mxfp4_1(lpr, ppl, full);
    case kFmtNvfp4: f = gateup_kernel_nvfp4_0(lpr, ppl, full); return f ? f : gateup_kernel_nvfp4_1(lpr, ppl, full);
    case kFmtAffine32:
      f = gateup_kernel_affine32_0(lpr, ppl, full);
      return f ? f : gateup_kernel_affine32_1(lpr, ppl, full);
    case kFmtAffine8: f = gateup_kernel_affine8_0(lpr, ppl, full); return f ? f : gateup_kernel_affine8_1(lpr, ppl, full);
    case kFmtMxfp8: f = gateup_kernel_mxfp8_0(lpr, ppl, full); return f ? f : gateup_kernel_mxfp8_1(lpr, ppl, full);
  }
  return nullptr;
}

const void* down_kernel_fmt(int fmt, int lpr, int ppl, bool full, int nt) {
  const void* f = nullptr;
  switch (fmt) {
    case kFmtMxfp4: f = down_kernel_mxfp4_0(lpr, ppl, full, nt); return f ? f : down_kernel_mxfp4_1(lpr, ppl, full, nt);
    case kFmtNvfp4: f = down_kernel_nvfp4_0(lpr, ppl, full, nt); return f ? f : down_kernel_nvfp4_1(lpr, ppl, full, nt);
    case kFmtAffine32:
      f = down_kernel_affine32_0(lpr, ppl, full, nt);
      return f ? f : down_kernel_affine32_1(lpr, ppl, full, nt);
    case kFmtAffine8:
      f = down_kernel_affine8_0(lpr, ppl, full, nt);
      return f ? f : down_kernel_affine8_1(lpr, ppl, full, nt);
    case kFmtMxfp8: f = down_kernel_mxfp8_0(lpr, ppl, full, nt); return f ? f : down_kernel_mxfp8_1(lpr, ppl, full, nt);
  }
  return nullptr;
}

}  // namespace moeq4
