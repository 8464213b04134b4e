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

constexpr int kThreads = 512;        // gate/up blocks: 8 waves sharing the staged activations
constexpr int kWaves = kThreads / 64;
constexpr int kDownThreads = 256;    // down blocks: 4 independent waves
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
// shared pieces
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint4 ld16(const unsigned char* base, uint32_t off) {
  return *reinterpret_cast<const uint4*>(base + off);
}
__device__ __forceinline__ uint32_t ld4(const unsigned char* base, uint32_t off) {
  return *reinterpret_cast<const uint32_t*>(base + off);
}
__device__ __forceinline__ uint32_t ld2(const unsigned char* base, uint32_t off) {
  return *reinterpret_cast<const uint16_t*>(base + off);
}

__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// D = sum over the 32 inputs of one 16-byte load of a_c * (M + q_c), with the
// activations a as 16 packed pairs in code order; M = 128 (bf16 pairs) or
// 1024 (fp16 pairs).
template <bool F16>
__device__ __forceinline__ float dot32(const uint4 w, const uint32_t (&av)[16], uint32_t magic, float d) {
  const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int wi = 0; wi < 4; ++wi) {
    uint32_t q[4];
    unpack_word(ww[wi], magic, q);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) d = F16 ? dot2_f16(q[kk], av[4 * wi + kk], d) : dot2_bf16(q[kk], av[4 * wi + kk], d);
  }
  return d;
}

// Scale and bias of the 64-input group that holds this lane's 32 inputs,
// packed as bf16 scale (low half) | bf16 bias (high half).
//
// Quad-shared form: the four lanes of a quad cover two consecutive groups;
// lane A of the quad loaded one dword (both groups) of array A, so two
// broadcasts and one byte permute give every lane its own pair.  `sel`
// picks the low (even group) or high (odd group) halves.
template <int AS, int AB>
__device__ __forceinline__ uint32_t quad_scale_bias(uint32_t q, uint32_t sel) {
  return __builtin_amdgcn_perm(quad_bcast<AB>(q), quad_bcast<AS>(q), sel);
}

// ---------------------------------------------------------------------------
// fused gate + up
// ---------------------------------------------------------------------------

// Packed weights of one gate/up work unit held by one lane: PPL positions x
// RG rows x {gate, up}, each a 16-byte load, plus scales and biases: with
// quad-shared loads one dword per (position, row) (array = lane % 4: gate
// scale, gate bias, up scale, up bias), otherwise one packed pair per
// (position, row, matrix).
template <int PPL, int RG>
struct GuFrag {
  uint4 w[PPL][RG][2];
  uint32_t sb[PPL][RG][2];
};

template <int PPL, int RG>
struct GuOffsets {
  uint32_t w[PPL][RG];   // byte offsets into the unit's packed codes
  uint32_t s[PPL][RG];   // byte offsets into the unit's scale / bias rows
};

template <int PPL, int RG, bool FULL, bool QS>
__device__ __forceinline__ void gu_load(const UnionArgs& a, size_t row0, int KU, int KG, int li, int lpr,
                                        const unsigned char* lane_sbase, const GuOffsets<PPL, RG>& o,
                                        GuFrag<PPL, RG>& f) {
  const unsigned char* wg = reinterpret_cast<const unsigned char*>(a.wg) + row0 * KU * 16;
  const unsigned char* wu = reinterpret_cast<const unsigned char*>(a.wu) + row0 * KU * 16;
  const size_t soff = row0 * KG * 2;
#pragma unroll
  for (int p = 0; p < PPL; ++p) {
    if (FULL || li + lpr * p < KU) {
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        f.w[p][r][0] = ld16(wg, o.w[p][r]);
        f.w[p][r][1] = ld16(wu, o.w[p][r]);
        if (QS) {
          f.sb[p][r][0] = ld4(lane_sbase + soff, o.s[p][r]);
        } else {
          const unsigned char* base = reinterpret_cast<const unsigned char*>(a.sg) + soff;
          f.sb[p][r][0] = ld2(base, o.s[p][r]) |
                          (ld2(reinterpret_cast<const unsigned char*>(a.bg) + soff, o.s[p][r]) << 16);
          f.sb[p][r][1] = ld2(reinterpret_cast<const unsigned char*>(a.su) + soff, o.s[p][r]) |
                          (ld2(reinterpret_cast<const unsigned char*>(a.bu) + soff, o.s[p][r]) << 16);
        }
      }
    }
  }
}

// One unit: gate and up of RG hidden rows of one distinct expert for every
// token routed to it, one token at a time (the unit's weights stay in
// registers); h = silu(gate) * up goes to hbuf[(slot0 + token rank) * I + row].
template <int LPR, int PPL, int RG, bool FULL, bool QS>
__device__ __forceinline__ void gu_compute(const UnionArgs& a, const GuFrag<PPL, RG>& f, uint32_t mask, int slot0,
                                           int row, int li, int KU, const uint4* act, const float* asum,
                                           uint32_t sel) {
  uint32_t sbv[PPL][RG][2];
#pragma unroll
  for (int p = 0; p < PPL; ++p)
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      if (QS) {
        sbv[p][r][0] = quad_scale_bias<0, 1>(f.sb[p][r][0], sel);
        sbv[p][r][1] = quad_scale_bias<2, 3>(f.sb[p][r][0], sel);
      } else {
        sbv[p][r][0] = f.sb[p][r][0];
        sbv[p][r][1] = f.sb[p][r][1];
      }
    }
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
      if (FULL || j < KU) {
        const uint4* xa = act + (size_t)t * 4 * KU + j;
        const uint4 x0 = xa[0], x1 = xa[KU], x2 = xa[2 * KU], x3 = xa[3 * KU];
        const uint32_t xv[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                                 x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
        const float xs = asum[(size_t)t * KU + j];
#pragma unroll
        for (int r = 0; r < RG; ++r)
#pragma unroll
          for (int mm = 0; mm < 2; ++mm) {
            const float d = dot32<false>(f.w[p][r][mm], xv, kMagicBytes, 0.0f);
            const float sc = bf16_lo_to_f32(sbv[p][r][mm]);
            const float bi = bf16_hi_to_f32(sbv[p][r][mm]) - 128.0f * sc;
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

template <int LPR, int PPL, bool FULL, bool QS>
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
      a.utab[i] = make_int4(s.uniq[i], (int)s.mask[i], s.off[i], 0);
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

  const int lane = tid & 63;
  const int wave = wave_uniform(tid >> 6);
  const int g = lane / LPR, li = lane % LPR;
  const int qa = li & 3;                  // this lane's array in the quad-shared scale loads
  const unsigned char* lane_sbase = reinterpret_cast<const unsigned char*>(
      qa == 0 ? (const void*)a.sg : qa == 1 ? (const void*)a.bg : qa == 2 ? (const void*)a.su : (const void*)a.bu);
  const uint32_t sel = ((li >> 1) & 1) ? 0x07060302u : 0x05040100u;
  GuOffsets<PPL, RG> o;
#pragma unroll
  for (int p = 0; p < PPL; ++p)
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      const int j = li + LPR * p;
      o.w[p][r] = (uint32_t)(((g * RG + r) * KU + j) * 16);
      const int grp = QS ? 2 * (li >> 2) + (LPR / 2) * p : (j >> 1);
      o.s[p][r] = (uint32_t)(((g * RG + r) * KG + grp) * 2);
    }
  const int upe = I / WROWS;                // wave units per expert
  const int nunits = u * upe;
  const int stride = gridDim.x * kWaves;
  int unit = blockIdx.x * kWaves + wave;

  // unit -> (distinct expert i, first row of the wave unit); units U, U + stride,
  // U + 2 stride, ... of this wave stream through a ring of three register
  // fragments: two in flight while the third is computed
  auto load = [&](int un, GuFrag<PPL, RG>& f) {
    const int i = un / upe;
    gu_load<PPL, RG, FULL, QS>(a, (size_t)wave_uniform(s.uniq[i]) * I + (un - i * upe) * WROWS, KU, KG, li, LPR,
                               lane_sbase, o, f);
  };
  auto compute = [&](int un, const GuFrag<PPL, RG>& f) {
    const int i = un / upe;
    gu_compute<LPR, PPL, RG, FULL, QS>(a, f, wave_uniform((int)s.mask[i]), wave_uniform(s.off[i]),
                                       (un - i * upe) * WROWS + g * RG, li, KU, act, asum, sel);
  };
  GuFrag<PPL, RG> f0, f1, f2;
  if (unit < nunits) load(unit, f0);
  if (unit + stride < nunits) load(unit + stride, f1);
  while (unit < nunits) {
    if (unit + 2 * stride < nunits) load(unit + 2 * stride, f2);
    compute(unit, f0);
    unit += stride;
    if (unit >= nunits) break;
    if (unit + 2 * stride < nunits) load(unit + 2 * stride, f0);
    compute(unit, f1);
    unit += stride;
    if (unit >= nunits) break;
    if (unit + 2 * stride < nunits) load(unit + 2 * stride, f1);
    compute(unit, f2);
    unit += stride;
  }
}

// ---------------------------------------------------------------------------
// down projection (per expert and token, router-weighted)
// ---------------------------------------------------------------------------

// RS rows x PPL positions of packed codes plus scales and biases: quad-shared
// (lane % 4 = 0, 1: scale, bias of row 2k; 2, 3: of row 2k + 1) or one packed
// pair per (row, position).
template <int PPL, int RS>
struct DnFrag {
  uint4 w[RS][PPL];
  uint32_t sb[RS][PPL];
};

template <int PPL, int RS>
struct DnOffsets {
  uint32_t w[RS][PPL];
  uint32_t s[RS][PPL];
};

template <int PPL, int RS, bool FULL, bool QS>
__device__ __forceinline__ void dn_load(const UnionArgs& a, size_t row0, int KU, int KG, int li, int lpr,
                                        const unsigned char* lane_sbase, const DnOffsets<PPL, RS>& o,
                                        DnFrag<PPL, RS>& f) {
  const unsigned char* wd = reinterpret_cast<const unsigned char*>(a.wd) + row0 * KU * 16;
  const size_t soff = row0 * KG * 2;
#pragma unroll
  for (int r = 0; r < RS; ++r)
#pragma unroll
    for (int p = 0; p < PPL; ++p)
      if (FULL || li + lpr * p < KU) {
        f.w[r][p] = ld16(wd, o.w[r][p]);
        if (QS) {
          if ((r & 1) == 0) f.sb[r][p] = ld4(lane_sbase + soff, o.s[r][p]);
        } else {
          f.sb[r][p] = ld2(reinterpret_cast<const unsigned char*>(a.sd) + soff, o.s[r][p]) |
                       (ld2(reinterpret_cast<const unsigned char*>(a.bd) + soff, o.s[r][p]) << 16);
        }
      }
}

// One step: RS rows of this lane group against the NT staged hidden vectors
// (fp16 pairs scaled by 2^k per token); each (row, token) result, times the
// token's router weight, goes to ys.
template <int LPR, int PPL, int RS, int NT, bool FULL, bool QS>
__device__ __forceinline__ void dn_step(const UnionArgs& a, const DnFrag<PPL, RS>& f, const uint32_t (&hv)[NT][PPL][16],
                                       const float (&hs)[NT][PPL], const float (&tw)[NT], int nt, int slot, int row0,
                                       int li, int KU, uint32_t sel) {
#pragma unroll
  for (int r = 0; r < RS; ++r) {
    float acc[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) acc[c] = 0.0f;
#pragma unroll
    for (int p = 0; p < PPL; ++p) {
      if (FULL || li + LPR * p < KU) {
        uint32_t sb;
        if (QS)
          sb = (r & 1) ? quad_scale_bias<2, 3>(f.sb[r & ~1][p], sel) : quad_scale_bias<0, 1>(f.sb[r][p], sel);
        else
          sb = f.sb[r][p];
        const float sc = bf16_lo_to_f32(sb);
        const float bi = bf16_hi_to_f32(sb) - 1024.0f * sc;
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          if (c < nt) {
            const float d = dot32<true>(f.w[r][p], hv[c][p], kMagicBytesF16, 0.0f);
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

template <int LPR, int PPL, bool FULL, bool QS>
__global__ __launch_bounds__(kDownThreads) void k_down(UnionArgs a) {
  constexpr int G = 64 / LPR;
  constexpr int RS = down_rows(G);       // a wave step covers G * RS rows
  constexpr int WSTEP = G * RS;
  constexpr int NT = kDownTokChunk;
  constexpr int NW = kDownThreads / 64;
  static_assert(!QS || RS % 2 == 0, "quad-shared scales pair rows");
  extern __shared__ __align__(16) unsigned char smem[];
  int4* utab = reinterpret_cast<int4*>(smem);
  const int H = a.H, I = a.I;
  const int KU = I >> 5, KG = I >> 6;
  const int tid = threadIdx.x;
  const int u = (int)a.hdr[2];
  for (int i = tid; i < u; i += blockDim.x) utab[i] = a.utab[i];
  __syncthreads();

  const int lane = tid & 63;
  const int wave = wave_uniform(tid >> 6);
  const int g = lane / LPR, li = lane % LPR;
  const int qa = li & 3;
  const unsigned char* lane_sbase =
      reinterpret_cast<const unsigned char*>((qa & 1) ? (const void*)a.bd : (const void*)a.sd);
  const uint32_t sel = ((li >> 1) & 1) ? 0x07060302u : 0x05040100u;
  DnOffsets<PPL, RS> o;
#pragma unroll
  for (int r = 0; r < RS; ++r)
#pragma unroll
    for (int p = 0; p < PPL; ++p) {
      const int j = li + LPR * p;
      o.w[r][p] = (uint32_t)(((g * RS + r) * KU + j) * 16);
      const int srow = QS ? (r & ~1) + (qa >> 1) : r;
      const int grp = QS ? 2 * (li >> 2) + (LPR / 2) * p : (j >> 1);
      o.s[r][p] = (uint32_t)(((g * RS + srow) * KG + grp) * 2);
    }

  // this wave's contiguous share of the (distinct expert, row step) sequence
  const int spe = H / WSTEP;
  const int total = u * spe;
  const int nwaves = gridDim.x * NW;
  const int per = (total + nwaves - 1) / nwaves;
  const int f_begin = min(total, (blockIdx.x * NW + wave) * per);
  const int f_end = min(total, f_begin + per);

  for (int f = f_begin; f < f_end;) {
    const int i = f / spe;
    const int seg_end = min(f_end, (i + 1) * spe);
    const int4 ent = utab[i];
    const int e = wave_uniform(ent.x), slot0 = wave_uniform(ent.z);
    const int ntok = __popc((uint32_t)wave_uniform(ent.y));
    const size_t ebase = (size_t)e * H;
    for (int t0 = 0; t0 < ntok; t0 += NT) {
      const int nt = min(NT, ntok - t0);
      // hidden vectors of up to NT tokens, each scaled by a power of two so
      // that its largest magnitude lies in [2^13, 2^14), rounded to fp16 pairs
      // in code order; hs = sum of the fp16 values per 32-input position
      uint32_t hv[NT][PPL][16];
      float hs[NT][PPL], tw[NT];
#pragma unroll
      for (int c = 0; c < NT; ++c) {
        const int slot = slot0 + t0 + (c < nt ? c : 0);
        float v[PPL][32];
        float mx = 0.0f;
#pragma unroll
        for (int p = 0; p < PPL; ++p) {
          const int j = li + LPR * p;
          if (FULL || j < KU) {
            const float4* src = reinterpret_cast<const float4*>(a.hbuf + (size_t)slot * I + 32 * j);
#pragma unroll
            for (int q4 = 0; q4 < 8; ++q4) {
              const float4 f4 = src[q4];
              v[p][4 * q4 + 0] = f4.x; v[p][4 * q4 + 1] = f4.y; v[p][4 * q4 + 2] = f4.z; v[p][4 * q4 + 3] = f4.w;
            }
          } else {
#pragma unroll
            for (int n = 0; n < 32; ++n) v[p][n] = 0.0f;
          }
#pragma unroll
          for (int n = 0; n < 32; ++n) mx = fmaxf(mx, fabsf(v[p][n]));
        }
        mx = wave_max(mx);
        const int ex = mx > 0.0f ? __builtin_amdgcn_frexp_expf(mx) : 0;
        const float up = __builtin_ldexpf(1.0f, 14 - ex);
        tw[c] = a.slot_w[slot] * __builtin_ldexpf(1.0f, ex - 14);
#pragma unroll
        for (int p = 0; p < PPL; ++p) {
          float sum = 0.0f;
#pragma unroll
          for (int wi = 0; wi < 4; ++wi) {
            _Float16 hb[8];
#pragma unroll
            for (int n = 0; n < 8; ++n) {
              hb[n] = (_Float16)(v[p][8 * wi + n] * up);
              sum += (float)hb[n];
            }
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
              hv[c][p][4 * wi + kk] = (uint32_t)__builtin_bit_cast(uint16_t, hb[pair_lo(kk)]) |
                                      ((uint32_t)__builtin_bit_cast(uint16_t, hb[pair_hi(kk)]) << 16);
          }
          hs[c][p] = sum;
        }
      }

      // steps st, st+1, ... of this segment stream through a ring of three
      // register fragments: two in flight while the third is computed
      auto load = [&](int sx, DnFrag<PPL, RS>& fr) {
        dn_load<PPL, RS, FULL, QS>(a, ebase + (size_t)(sx - i * spe) * WSTEP, KU, KG, li, LPR, lane_sbase, o, fr);
      };
      auto step = [&](int sx, const DnFrag<PPL, RS>& fr) {
        dn_step<LPR, PPL, RS, NT, FULL, QS>(a, fr, hv, hs, tw, nt, slot0 + t0, (sx - i * spe) * WSTEP + g * RS, li,
                                            KU, sel);
      };
      DnFrag<PPL, RS> f0, f1, f2;
      int st = f;
      load(st, f0);
      if (st + 1 < seg_end) load(st + 1, f1);
#pragma unroll 1
      while (st < seg_end) {
        if (st + 2 < seg_end) load(st + 2, f2);
        step(st, f0);
        if (++st >= seg_end) break;
        if (st + 2 < seg_end) load(st + 2, f0);
        step(st, f1);
        if (++st >= seg_end) break;
        if (st + 2 < seg_end) load(st + 2, f1);
        step(st, f2);
        ++st;
      }
    }
    f = seg_end;
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

template <int LPR, int PPL, bool FULL, bool QS>
struct GateUpK {
  static const void* fn() { return reinterpret_cast<const void*>(&k_gateup<LPR, PPL, FULL, QS>); }
};
template <int LPR, int PPL, bool FULL, bool QS>
struct DownK {
  static const void* fn() { return reinterpret_cast<const void*>(&k_down<LPR, PPL, FULL, QS>); }
};

// QS (quad-shared scale loads) needs lane groups of at least 4 and an even
// number of 64-input groups per row, so that a quad's dword never passes the
// row's end.
template <template <int, int, bool, bool> class K>
const void* pick_kernel(int lpr, int ppl, bool full, bool qs, bool down) {
#define MOEQ4_CASE(L_, P_)                                                                               \
  if (lpr == L_ && ppl == P_)                                                                            \
    return full ? (qs && L_ >= 4 ? K<L_, P_, true, (L_ >= 4)>::fn() : K<L_, P_, true, false>::fn())      \
                : (qs && L_ >= 4 ? K<L_, P_, false, (L_ >= 4)>::fn() : K<L_, P_, false, false>::fn());
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

int blocks_per_cu(const void* fn, int threads, size_t lds) {
  static OccCache cache[64];
  static int n = 0;
  for (int c = 0; c < n; ++c)
    if (cache[c].fn == fn && cache[c].lds == lds) return cache[c].blocks;
  int b = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, fn, threads, lds) != hipSuccess || b < 1) b = 1;
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
    const void* fn = pick_kernel<GateUpK>(lpr, ppl, lpr * ppl == KU, (a.H / 64) % 2 == 0, false);
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
    const int KU = a.I / 32;
    const int lpr = lanes_per_row(KU), ppl = positions_per_lane(KU, lpr, true);
    const size_t lds = align16((size_t)16 * P);
    const void* fn = pick_kernel<DownK>(lpr, ppl, lpr * ppl == KU, (a.I / 64) % 2 == 0, true);
    if (!fn || lds > kMaxLds) return MOE_Q4_ERR_UNSUPPORTED;
    const int groups = 64 / lpr;
    const int wstep = groups * down_rows(groups);
    const int steps = u_max * (a.H / wstep);
    constexpr int nw = kDownThreads / 64;
    int grid = num_cu * blocks_per_cu(fn, kDownThreads, lds);
    const int need = (steps + nw - 1) / nw;
    if (grid > need) grid = need;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(reinterpret_cast<void (*)(UnionArgs)>(const_cast<void*>(fn)), dim3(grid),
                       dim3(kDownThreads), lds, stream, a);
    if (hipGetLastError() != hipSuccess) return MOE_Q4_ERR_LAUNCH;
    dim3 cgrid((a.H / 4 + 255) / 256, a.L);
    hipLaunchKernelGGL(k_combine, cgrid, dim3(256), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return MOE_Q4_ERR_LAUNCH;
  }
  return MOE_Q4_OK;
}

}  // namespace moeq4
