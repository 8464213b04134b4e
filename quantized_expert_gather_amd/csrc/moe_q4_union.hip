// Union path of the SwitchGLU-q4 MoE layer for gfx950 (MI355X).
//
// Kernels (one forward = gateup -> down -> combine on one stream):
//   k_route_union  the distinct experts of the L*k routes, their token masks,
//                  summed router weights and the slot -> distinct-id map
//                  (exported on its own for bit-exact checks).
//   k_gateup       every block builds the route union and stages the bf16
//                  activations of all L tokens in LDS once; then each wave,
//                  with no further barriers, streams work units (one distinct
//                  expert, a few hidden rows) with the next unit's packed
//                  gate and up weights already in flight, computes gate and up
//                  for every token routed to that expert in one pass, and
//                  writes h = silu(gate) * up in fp32.  Block 0 also writes
//                  the per-expert and per-token tables the later kernels read.
//   k_down         each wave streams units (one distinct expert, 64 output
//                  rows): the expert's hidden vectors are loaded once per unit
//                  into registers as exact bf16 hi + lo pairs, the down rows
//                  stream through with the next rows in flight, and each
//                  (expert, token) output, times the token's router weight, is
//                  written per pair.
//   k_combine      out[t] = sum of token t's per-pair outputs in ascending
//                  expert order (deterministic; no floating-point atomics).
//
// Sources (web pages): streaming every distinct routed expert once and
// applying it to each position routed to it is the union gather of the mlx
// discussion "Small-L fused expert gather for fine-grained MoE decode"
// (implication 1 of the overlap section); running gate and up in one pass with
// SiLU on the gate before the product follows the splash PR "perf: Apple7/8
// MoE gate and up in one decode pass" (section "What changed") and the
// SwitchGLU order of the mlx issue "gather_qmm at M=1 streams 4-bit expert
// weights at ~half the bandwidth of M=4" (moe_bench script).
//
// Inner product with affine codes.  For the 32 consecutive inputs c of one
// 16-byte load (one half of a 64-input (scale s, bias b) group):
//     sum_c a_c (s q_c + b) = s * D + (b - 128 s) * A,
//     D = sum_c a_c (128 + q_c),  A = sum_c a_c,
// where 128 + q_c is built exactly as bf16 by OR-ing the nibble into the
// mantissa of 128.0, and D accumulates with bf16 dot2 in fp32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_q4.h"
#include "moe_q4_device.h"
#include "moe_q4_internal.h"

namespace moeq4 {

constexpr int kThreads = 512;        // 8 waves per block
constexpr int kWaves = kThreads / 64;
constexpr int kDownUnitRows = 64;    // output rows of one down work unit
constexpr int kDownTokChunk = 2;     // tokens per register pass in down

// hidden rows per lane group in one gate/up unit (fewer when a row needs
// several 16-byte positions per lane, to keep two units in registers)
constexpr int gateup_rows(int ppl) { return ppl == 1 ? 2 : 1; }
// output rows per lane group in one down step
constexpr int down_rows(int groups) { return groups * 4 <= kDownUnitRows ? 4 : kDownUnitRows / groups; }

// ---------------------------------------------------------------------------
// route union (exported)
// ---------------------------------------------------------------------------

__device__ __forceinline__ void carve_union(unsigned char* base, int E, int P, UnionLds& s) {
  const int EW = (E + 31) >> 5;
  s.bitmap = reinterpret_cast<uint32_t*>(base);
  s.scan = reinterpret_cast<int32_t*>(s.bitmap + EW);
  s.uniq = s.scan + EW;
  s.mask = reinterpret_cast<uint32_t*>(s.uniq + P);
  s.off = reinterpret_cast<int32_t*>(s.mask + P);
  s.scal = s.off + P + 1;
}

__global__ __launch_bounds__(256) void k_route_union(const int32_t* __restrict__ ids, const float* __restrict__ tw,
                                                     int L, int k, int E, int32_t* __restrict__ u_out,
                                                     int32_t* __restrict__ uniq_ids, uint32_t* __restrict__ tok_mask,
                                                     float* __restrict__ uniq_w, int32_t* __restrict__ slot_to_uniq,
                                                     int u_max) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int P = L * k;
  UnionLds s;
  carve_union(smem, E, P, s);
  build_union(ids, P, k, E, s);
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
    if (i < u && ((s.mask[i] >> t) & 1u)) v = token_expert_weight(ids, tw, t, k, s.uniq[i]);
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
// fused gate + up
// ---------------------------------------------------------------------------

// Packed weights of one gate/up work unit held by one lane: PPL positions x
// RG rows x {gate, up}, each a 16-byte load plus its (scale, bias) pair.
template <int PPL, int RG>
struct GuFrag {
  uint4 w[PPL][RG][2];
  uint32_t sb[PPL][RG][2];  // bf16 scale (low half) | bf16 bias (high half)
};

template <int LPR, int PPL, int RG>
__device__ __forceinline__ void gu_load(const UnionArgs& a, int e, int row, int li, int KU, int KG,
                                        GuFrag<PPL, RG>& f) {
#pragma unroll
  for (int p = 0; p < PPL; ++p) {
    const int j = li + LPR * p;
    if (j < KU) {
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        const size_t rr = (size_t)e * a.I + row + r;
        f.w[p][r][0] = reinterpret_cast<const uint4*>(a.wg)[rr * KU + j];
        f.w[p][r][1] = reinterpret_cast<const uint4*>(a.wu)[rr * KU + j];
        const size_t g = rr * KG + (j >> 1);
        f.sb[p][r][0] = (uint32_t)a.sg[g] | ((uint32_t)a.bg[g] << 16);
        f.sb[p][r][1] = (uint32_t)a.su[g] | ((uint32_t)a.bu[g] << 16);
      }
    }
  }
}

// One unit: gate and up rows [row, row + RG) of distinct expert i for every
// token routed to it, one token at a time (the unit's weights stay in
// registers); h written to hbuf[(slot0 + token rank) * I + row].
template <int LPR, int PPL, int RG>
__device__ __forceinline__ void gu_compute(const UnionArgs& a, const GuFrag<PPL, RG>& f, uint32_t mask, int slot0,
                                           int row, int li, int KU, const uint4* act, const float* asum) {
  uint32_t m = mask;
  for (int c = 0; m; ++c) {
    const int t = __builtin_ctz(m);
    m &= m - 1u;
    float acc[RG][2];
#pragma unroll
    for (int r = 0; r < RG; ++r) acc[r][0] = acc[r][1] = 0.0f;
#pragma unroll
    for (int p = 0; p < PPL; ++p) {
      const int j = li + LPR * p;
      if (j < KU) {
        const uint4* xa = act + (size_t)t * 4 * KU + j;
        const uint4 x0 = xa[0], x1 = xa[KU], x2 = xa[2 * KU], x3 = xa[3 * KU];
        const uint32_t xv[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                                 x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
        const float xs = asum[(size_t)t * KU + j];
#pragma unroll
        for (int r = 0; r < RG; ++r)
#pragma unroll
          for (int mm = 0; mm < 2; ++mm) {
            const uint4 w = f.w[p][r][mm];
            uint32_t q[16];
            unpack_word(w.x, q + 0);
            unpack_word(w.y, q + 4);
            unpack_word(w.z, q + 8);
            unpack_word(w.w, q + 12);
            float d = 0.0f;
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) d = dot2_bf16(q[kk], xv[kk], d);
            const float sc = bf16_lo_to_f32(f.sb[p][r][mm]);
            const float bi = bf16_hi_to_f32(f.sb[p][r][mm]) - 128.0f * sc;
            acc[r][mm] += sc * d + bi * xs;
          }
      }
    }
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      const float gt = group_sum<LPR>(acc[r][0]);
      const float up = group_sum<LPR>(acc[r][1]);
      if (li == 0) a.hbuf[(size_t)(slot0 + c) * a.I + row + r] = gt / (1.0f + expf(-gt)) * up;
    }
  }
}

template <int LPR, int PPL>
__global__ __launch_bounds__(kThreads) void k_gateup(UnionArgs a) {
  constexpr int G = 64 / LPR;           // lane groups per wave
  constexpr int RG = gateup_rows(PPL);
  constexpr int WROWS = G * RG;         // hidden rows of one wave unit
  extern __shared__ __align__(16) unsigned char smem[];
  const int H = a.H, I = a.I, k = a.k, L = a.L, E = a.E;
  const int P = L * k;
  const int KU = H >> 5, KG = H >> 6;
  uint4* act = reinterpret_cast<uint4*>(smem + a.lds_act);      // [L][4][KU] bf16 pairs in code order
  float* asum = reinterpret_cast<float*>(smem + a.lds_asum);     // [L][KU] sums of the 32 inputs
  UnionLds s;
  carve_union(smem + a.lds_union, E, P, s);

  // stage all tokens' activations (independent of the union; overlaps it)
  const int tid = threadIdx.x;
  for (int it = tid; it < L * KU; it += blockDim.x) {
    const int t = it / KU, j = it - t * KU;
    const uint4* xs = reinterpret_cast<const uint4*>(a.x + (size_t)t * H) + 4 * j;
    float sum = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 v = xs[c];
      sum = sum8_bf16(v, sum);
      act[((size_t)t * 4 + c) * KU + j] = pair_activations(v);
    }
    asum[(size_t)t * KU + j] = sum;
  }
  build_union(a.ids, P, k, E, s);  // ends with a barrier
  const int u = s.scal[0];

  if (blockIdx.x == 0) {
    // tables for the down and combine kernels
    if (tid == 0) {
      a.hdr[0] = s.scal[1] ? MOE_Q4_DEV_BAD_ID : 0u;  // status of this call
      a.hdr[1] = MOE_Q4_PATH_UNION;
      a.hdr[2] = (uint32_t)u;
    }
    for (int i = tid; i < u; i += blockDim.x) {
      const int4 ent = make_int4(s.uniq[i], (int)s.mask[i], s.off[i], 0);
      a.utab[i] = ent;
      uint32_t m = s.mask[i];
      for (int c = 0; m; ++c) {
        const int t = __builtin_ctz(m);
        m &= m - 1u;
        a.slot_w[s.off[i] + c] = token_expert_weight(a.ids, a.tw, t, k, s.uniq[i]);
      }
    }
    for (int t = tid; t < L; t += blockDim.x) {
      int c = 0;
      for (int i = 0; i < u; ++i) {
        const uint32_t m = s.mask[i];
        if ((m >> t) & 1u) a.tslot[t * k + c++] = s.off[i] + __popc(m & ((1u << t) - 1u));
      }
      a.tcount[t] = c;
    }
  }

  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane / LPR, li = lane % LPR;
  const int upe = I / WROWS;                // wave units per expert
  const int nunits = u * upe;
  const int stride = gridDim.x * kWaves;
  int unit = blockIdx.x * kWaves + wave;

  GuFrag<PPL, RG> fa, fb;
  auto unit_row = [&](int un, int& i) {
    i = un / upe;
    return (un - i * upe) * WROWS + g * RG;
  };
  int ia, ib;
  if (unit < nunits) {
    const int row = unit_row(unit, ia);
    gu_load<LPR, PPL, RG>(a, s.uniq[ia], row, li, KU, KG, fa);
  }
  while (unit < nunits) {
    int nxt = unit + stride;
    if (nxt < nunits) {
      const int row = unit_row(nxt, ib);
      gu_load<LPR, PPL, RG>(a, s.uniq[ib], row, li, KU, KG, fb);
    }
    {
      const int row = unit_row(unit, ia);
      gu_compute<LPR, PPL, RG>(a, fa, s.mask[ia], s.off[ia], row, li, KU, act, asum);
    }
    unit = nxt;
    if (unit >= nunits) break;
    nxt = unit + stride;
    if (nxt < nunits) {
      const int row = unit_row(nxt, ia);
      gu_load<LPR, PPL, RG>(a, s.uniq[ia], row, li, KU, KG, fa);
    }
    {
      const int row = unit_row(unit, ib);
      gu_compute<LPR, PPL, RG>(a, fb, s.mask[ib], s.off[ib], row, li, KU, act, asum);
    }
    unit = nxt;
  }
}

// ---------------------------------------------------------------------------
// down projection (per expert and token, router-weighted)
// ---------------------------------------------------------------------------

template <int PPL, int RS>
struct DnFrag {
  uint4 w[RS][PPL];
  uint32_t sb[RS][PPL];
};

template <int LPR, int PPL, int RS>
__device__ __forceinline__ void dn_load(const UnionArgs& a, int e, int row, int li, int KU, int KG,
                                        DnFrag<PPL, RS>& f) {
#pragma unroll
  for (int r = 0; r < RS; ++r) {
    const size_t rr = (size_t)e * a.H + row + r;
#pragma unroll
    for (int p = 0; p < PPL; ++p) {
      const int j = li + LPR * p;
      if (j < KU) {
        f.w[r][p] = reinterpret_cast<const uint4*>(a.wd)[rr * KU + j];
        const size_t gg = rr * KG + (j >> 1);
        f.sb[r][p] = (uint32_t)a.sd[gg] | ((uint32_t)a.bd[gg] << 16);
      }
    }
  }
}

// One step of a down unit: RS rows of this lane group against the NT staged
// hidden vectors; each (row, token) result times the token's router weight
// goes to ys.
template <int LPR, int PPL, int RS, int NT>
__device__ __forceinline__ void dn_step(const UnionArgs& a, const DnFrag<PPL, RS>& f, const uint32_t (&hh)[NT][PPL][16],
                                       const uint32_t (&hl)[NT][PPL][16], const float (&hs)[NT][PPL],
                                       const float (&tw)[NT], int nt, int slot, int row0, int li, int KU) {
#pragma unroll
  for (int r = 0; r < RS; ++r) {
    float acc[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) acc[c] = 0.0f;
#pragma unroll
    for (int p = 0; p < PPL; ++p) {
      const int j = li + LPR * p;
      if (j < KU) {
        const uint4 w = f.w[r][p];
        uint32_t q[16];
        unpack_word(w.x, q + 0);
        unpack_word(w.y, q + 4);
        unpack_word(w.z, q + 8);
        unpack_word(w.w, q + 12);
        const float sc = bf16_lo_to_f32(f.sb[r][p]);
        const float bi = bf16_hi_to_f32(f.sb[r][p]) - 128.0f * sc;
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          if (c < nt) {
            float d = 0.0f;
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) d = dot2_bf16(q[kk], hh[c][p][kk], d);
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) d = dot2_bf16(q[kk], hl[c][p][kk], d);
            acc[c] += sc * d + bi * hs[c][p];
          }
        }
      }
    }
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      if (c < nt) {
        const float y = group_sum<LPR>(acc[c]);
        if (li == 0) a.ys[(size_t)(slot + c) * a.H + row0 + r] = tw[c] * y;
      }
    }
  }
}

template <int LPR, int PPL>
__global__ __launch_bounds__(kThreads) void k_down(UnionArgs a) {
  constexpr int G = 64 / LPR;
  constexpr int RS = down_rows(G);       // a wave step covers G * RS rows (<= 64)
  constexpr int WSTEP = G * RS;
  constexpr int NSTEP = kDownUnitRows / WSTEP;
  constexpr int NT = kDownTokChunk;
  static_assert(NSTEP >= 1 && NSTEP * WSTEP == kDownUnitRows, "down step shape");
  extern __shared__ __align__(16) unsigned char smem[];
  int4* utab = reinterpret_cast<int4*>(smem);
  const int H = a.H, I = a.I;
  const int KU = I >> 5, KG = I >> 6;
  const int tid = threadIdx.x;
  const int u = (int)a.hdr[2];
  for (int i = tid; i < u; i += blockDim.x) utab[i] = a.utab[i];
  __syncthreads();

  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane / LPR, li = lane % LPR;
  const int upe = H / kDownUnitRows;
  const int nunits = u * upe;
  const int stride = gridDim.x * kWaves;

  for (int unit = blockIdx.x * kWaves + wave; unit < nunits; unit += stride) {
    const int i = unit / upe;
    const int rbase = (unit - i * upe) * kDownUnitRows + g * RS;
    const int4 ent = utab[i];
    const int e = ent.x, slot0 = ent.z;
    const int ntok = __popc((uint32_t)ent.y);
    for (int t0 = 0; t0 < ntok; t0 += NT) {
      const int nt = min(NT, ntok - t0);
      // hidden vectors of up to NT tokens -> exact bf16 hi/lo pairs in code
      // order, plus the sum of hi + lo over each 32-input position
      uint32_t hh[NT][PPL][16], hl[NT][PPL][16];
      float hs[NT][PPL], tw[NT];
#pragma unroll
      for (int c = 0; c < NT; ++c) {
        const int slot = slot0 + t0 + (c < nt ? c : 0);
        tw[c] = a.slot_w[slot];
#pragma unroll
        for (int p = 0; p < PPL; ++p) {
          const int j = li + LPR * p;
          float sum = 0.0f;
          if (j < KU) {
            const float4* src = reinterpret_cast<const float4*>(a.hbuf + (size_t)slot * I + 32 * j);
#pragma unroll
            for (int wi = 0; wi < 4; ++wi) {
              const float4 v0 = src[2 * wi], v1 = src[2 * wi + 1];
              const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
              uint32_t hb[8], lb[8];
#pragma unroll
              for (int n = 0; n < 8; ++n) {
                hb[n] = f32_to_bf16_rne(v[n]);
                const float hf = __uint_as_float(hb[n] << 16);
                lb[n] = f32_to_bf16_rne(v[n] - hf);
                sum += hf + __uint_as_float(lb[n] << 16);
              }
#pragma unroll
              for (int kk = 0; kk < 4; ++kk) {
                hh[c][p][4 * wi + kk] = hb[kk] | (hb[kk + 4] << 16);
                hl[c][p][4 * wi + kk] = lb[kk] | (lb[kk + 4] << 16);
              }
            }
          }
          hs[c][p] = sum;
        }
      }

      DnFrag<PPL, RS> fa, fb;
      dn_load<LPR, PPL, RS>(a, e, rbase, li, KU, KG, fa);
#pragma unroll 1
      for (int st = 0; st < NSTEP; st += 2) {
        if (st + 1 < NSTEP) dn_load<LPR, PPL, RS>(a, e, rbase + (st + 1) * WSTEP, li, KU, KG, fb);
        dn_step<LPR, PPL, RS, NT>(a, fa, hh, hl, hs, tw, nt, slot0 + t0, rbase + st * WSTEP, li, KU);
        if (st + 1 >= NSTEP) break;
        if (st + 2 < NSTEP) dn_load<LPR, PPL, RS>(a, e, rbase + (st + 2) * WSTEP, li, KU, KG, fa);
        dn_step<LPR, PPL, RS, NT>(a, fb, hh, hl, hs, tw, nt, slot0 + t0, rbase + (st + 1) * WSTEP, li, KU);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// combine: out[t, m] = sum over t's pairs (ascending expert) of ys[pair, m]
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_combine(UnionArgs a) {
  const int H = a.H, k = a.k;
  const int n4 = H >> 2;
  const int it = blockIdx.x * blockDim.x + threadIdx.x;  // one float4 of one token
  const int t = blockIdx.y;
  if (it >= n4) return;
  const int cnt = a.tcount[t];
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int c = 0; c < cnt; ++c) {
    const float4 v = reinterpret_cast<const float4*>(a.ys + (size_t)a.tslot[t * k + c] * H)[it];
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

template <int LPR, int PPL>
struct GateUpK {
  static const void* fn() { return reinterpret_cast<const void*>(&k_gateup<LPR, PPL>); }
};
template <int LPR, int PPL>
struct DownK {
  static const void* fn() { return reinterpret_cast<const void*>(&k_down<LPR, PPL>); }
};

template <template <int, int> class K>
const void* pick_kernel(int lpr, int ppl, bool down) {
#define MOEQ4_CASE(L_, P_) \
  if (lpr == L_ && ppl == P_) return K<L_, P_>::fn();
  if (!down) {
    MOEQ4_CASE(64, 1) MOEQ4_CASE(64, 2) MOEQ4_CASE(64, 3) MOEQ4_CASE(64, 4) MOEQ4_CASE(64, 6) MOEQ4_CASE(64, 8)
  } else {
    MOEQ4_CASE(64, 1) MOEQ4_CASE(64, 2) MOEQ4_CASE(64, 4)
  }
  MOEQ4_CASE(32, 1) MOEQ4_CASE(16, 1) MOEQ4_CASE(8, 1) MOEQ4_CASE(4, 1) MOEQ4_CASE(2, 1)
#undef MOEQ4_CASE
  return nullptr;
}

size_t align16(size_t v) { return (v + 15) & ~size_t(15); }

size_t union_lds(int E, int P) { return (size_t)4 * (2 * ((E + 31) >> 5) + 3 * P + 1 + 2); }

// gate/up LDS: activations of all L tokens | their 32-input sums | route union
size_t gateup_lds_layout(UnionArgs& a) {
  const int KU = a.H / 32;
  size_t off = 0;
  a.lds_act = off;   off = align16(off + (size_t)a.L * 4 * KU * 16);
  a.lds_asum = off;  off = align16(off + (size_t)a.L * KU * 4);
  a.lds_union = off; off = align16(off + union_lds(a.E, a.L * a.k));
  return off;
}

constexpr size_t kMaxLds = 160 * 1024;

struct OccCache {
  const void* fn;
  size_t lds;
  int blocks;
};

int blocks_per_cu(const void* fn, size_t lds) {
  static OccCache cache[64];
  static int n = 0;
  for (int c = 0; c < n; ++c)
    if (cache[c].fn == fn && cache[c].lds == lds) return cache[c].blocks;
  int b = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, fn, kThreads, lds) != hipSuccess || b < 1) b = 1;
  if (n < 64) cache[n++] = OccCache{fn, lds, b};
  return b;
}

}  // namespace

size_t union_lds_bytes_max(int L, int k, int E, int H, int I) {
  UnionArgs a{};
  a.L = L; a.k = k; a.E = E; a.H = H; a.I = I;
  return gateup_lds_layout(a);
}

bool union_shape_supported(int L, int k, int E, int H, int I) {
  const int lg = lanes_per_row(H / 32), ld = lanes_per_row(I / 32);
  if (!positions_per_lane(H / 32, lg, false) || !positions_per_lane(I / 32, ld, true)) return false;
  if ((I % (gateup_rows(positions_per_lane(H / 32, lg, false)) * (64 / lg))) != 0) return false;
  return union_lds_bytes_max(L, k, E, H, I) <= kMaxLds && (size_t)4 * 16 * (L * k) <= kMaxLds;
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
    const int KU = a.H / 32;
    const int lpr = lanes_per_row(KU), ppl = positions_per_lane(KU, lpr, false);
    const size_t lds = gateup_lds_layout(a);
    const void* fn = pick_kernel<GateUpK>(lpr, ppl, false);
    if (!fn || lds > kMaxLds) return MOE_Q4_ERR_UNSUPPORTED;
    const int wunits = u_max * (a.I / (gateup_rows(ppl) * (64 / lpr)));
    int grid = num_cu * blocks_per_cu(fn, lds);
    const int need = (wunits + kWaves - 1) / kWaves;
    if (grid > need) grid = need;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(reinterpret_cast<void (*)(UnionArgs)>(const_cast<void*>(fn)), dim3(grid), dim3(kThreads),
                       lds, stream, a);
    if (hipGetLastError() != hipSuccess) return MOE_Q4_ERR_LAUNCH;
  }
  if (stages & MOE_Q4_STAGE_DOWN) {
    UnionArgs a = base;
    const int KU = a.I / 32;
    const int lpr = lanes_per_row(KU), ppl = positions_per_lane(KU, lpr, true);
    const size_t lds = align16((size_t)16 * P);
    const void* fn = pick_kernel<DownK>(lpr, ppl, true);
    if (!fn || lds > kMaxLds) return MOE_Q4_ERR_UNSUPPORTED;
    const int wunits = u_max * (a.H / kDownUnitRows);
    int grid = num_cu * blocks_per_cu(fn, lds);
    const int need = (wunits + kWaves - 1) / kWaves;
    if (grid > need) grid = need;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(reinterpret_cast<void (*)(UnionArgs)>(const_cast<void*>(fn)), dim3(grid), dim3(kThreads),
                       lds, stream, a);
    if (hipGetLastError() != hipSuccess) return MOE_Q4_ERR_LAUNCH;
    dim3 cgrid((a.H / 4 + 255) / 256, a.L);
    hipLaunchKernelGGL(k_combine, cgrid, dim3(256), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return MOE_Q4_ERR_LAUNCH;
  }
  return MOE_Q4_OK;
}

}  // namespace moeq4
