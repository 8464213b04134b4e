// Kernel templates of the union path of the SwitchGLU-q4 MoE layer for gfx950
// (MI355X).  Internal header: the instantiation units include it.
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
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_q4.h"
#include "moe_q4_device.h"
#include "moe_q4_internal.h"
#include "moe_q4_union_mfma.h"

namespace moeq4 {

constexpr int kThreads = 512;        // gate/up blocks: 8 waves sharing the staged activations
constexpr int kWaves = kThreads / 64;
constexpr int kDownUnitRows = 64;    // output rows of one down step, at most

// hidden rows per lane group in one gate/up unit (fewer when a row needs
// several 16-byte positions per lane, to keep two units in registers)
constexpr int gateup_rows(int ppl) { return ppl == 1 ? 2 : 1; }
// output rows per lane group in one down step
constexpr int down_rows(int groups) { return groups * 4 <= kDownUnitRows ? 4 : kDownUnitRows / groups; }

// Carves the route-union LDS arrays out of `base` (layout of build_union).
__device__ __forceinline__ void carve_union(unsigned char* base, int E, int P, UnionLds& s) {
  const int EW = (E + 31) >> 5;
  s.bitmap = reinterpret_cast<uint32_t*>(base);
  s.scan = reinterpret_cast<int32_t*>(s.bitmap + EW);
  s.uniq = s.scan + EW;
  s.mask = reinterpret_cast<uint32_t*>(s.uniq + P);
  s.off = reinterpret_cast<int32_t*>(s.mask + P);
  s.scal = s.off + P + 1;
  s.ids = s.scal + 2;
  s.tw = reinterpret_cast<float*>(s.ids + P);
}

// ---------------------------------------------------------------------------
// shared pieces
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t ld4(const unsigned char* base, uint32_t off) {
  return *reinterpret_cast<const uint32_t*>(base + off);
}

__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Marks the registers of a prefetched fragment as used here, so the wait for
// its loads lands at this point and not inside the compute loop that follows.
__device__ __forceinline__ void touch(const uint4& v) { asm volatile("" ::"v"(v.x), "v"(v.y), "v"(v.z), "v"(v.w)); }
__device__ __forceinline__ void touch(uint32_t v) { asm volatile("" ::"v"(v)); }

// A copy of a weight fragment that the compiler cannot see through: the
// values derived from it (unpacked codes, converted pairs) are recomputed at
// each use instead of being kept live across a token loop.  With many
// positions per lane those derived values would take more registers than
// the load ring itself and spill.
template <bool OPAQUE>
__device__ __forceinline__ uint4 opaque(uint4 v) {
  if constexpr (OPAQUE) asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
  return v;
}
// positions per lane from which the gate/up kernel recomputes unpacked codes
// per token rather than keep them
constexpr int kGuOpaquePpl = 4;

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

// Loads unit `un` (or nothing, with zero-range descriptors, when !valid).
// Loads the unit whose first row is row0 (plain loads from a wave-uniform
// row base plus per-lane offsets).
template <int PPL, int RG, bool FULL, bool QS, int FMT = kFmtAffine>
__device__ __forceinline__ void gu_load(const UnionArgs& a, size_t row0, int nrows, int KU, int KG, int li, int lpr,
                                        const unsigned char* lane_sbase, const GuOffsets<PPL, RG>& o,
                                        GuFrag<PPL, RG>& f) {
  if constexpr (fmt_fp4(FMT) || FMT == kFmtMxfp8) {
    // scale bytes of a row: two E4M3 per position (nvfp4), one E8M0 per 32
    // inputs (mxfp4: per position; mxfp8: per two positions); packed gate
    // low, up high
    const size_t srow = FMT == kFmtNvfp4 ? (size_t)KU * 2 : FMT == kFmtMxfp8 ? (size_t)(KU >> 1) : (size_t)KU;
    const unsigned char* wg = reinterpret_cast<const unsigned char*>(a.wg) + row0 * KU * 16;
    const unsigned char* wu = reinterpret_cast<const unsigned char*>(a.wu) + row0 * KU * 16;
    const unsigned char* eg = reinterpret_cast<const unsigned char*>(a.sg) + row0 * srow;
    const unsigned char* eu = reinterpret_cast<const unsigned char*>(a.su) + row0 * srow;
#pragma unroll
    for (int p = 0; p < PPL; ++p) {
      if (FULL || li + lpr * p < KU) {
#pragma unroll
        for (int r = 0; r < RG; ++r) {
          f.w[p][r][0] = ld16_nt(wg + o.w[p][r]);
          f.w[p][r][1] = ld16_nt(wu + o.w[p][r]);
          if constexpr (FMT == kFmtNvfp4)
            f.sb[p][r][0] = (uint32_t)*reinterpret_cast<const uint16_t*>(eg + o.s[p][r]) |
                            ((uint32_t)*reinterpret_cast<const uint16_t*>(eu + o.s[p][r]) << 16);
          else
            f.sb[p][r][0] = (uint32_t)eg[o.s[p][r]] | ((uint32_t)eu[o.s[p][r]] << 8);
        }
      }
    }
    (void)nrows; (void)KG; (void)lane_sbase;
    return;
  }
  const uint32_t sbb = (uint32_t)(nrows * KG * 2);
  const unsigned char* wg = reinterpret_cast<const unsigned char*>(a.wg) + row0 * KU * 16;
  const unsigned char* wu = reinterpret_cast<const unsigned char*>(a.wu) + row0 * KU * 16;
  const size_t soff = row0 * KG * 2;
#pragma unroll
  for (int p = 0; p < PPL; ++p) {
    if (FULL || li + lpr * p < KU) {
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        f.w[p][r][0] = ld16_nt(wg + o.w[p][r]);
        f.w[p][r][1] = ld16_nt(wu + o.w[p][r]);
        if (QS) {
          f.sb[p][r][0] = ld4(lane_sbase + soff, o.s[p][r]);
        } else {
          const rsrc_t sg = make_rsrc(reinterpret_cast<const unsigned char*>(a.sg) + row0 * KG * 2, sbb);
          const rsrc_t bg = make_rsrc(reinterpret_cast<const unsigned char*>(a.bg) + row0 * KG * 2, sbb);
          const rsrc_t su = make_rsrc(reinterpret_cast<const unsigned char*>(a.su) + row0 * KG * 2, sbb);
          const rsrc_t bu = make_rsrc(reinterpret_cast<const unsigned char*>(a.bu) + row0 * KG * 2, sbb);
          f.sb[p][r][0] = bld2(sg, o.s[p][r]) | (bld2(bg, o.s[p][r]) << 16);
          f.sb[p][r][1] = bld2(su, o.s[p][r]) | (bld2(bu, o.s[p][r]) << 16);
        }
      }
    }
  }
}

// One unit: gate and up of RG hidden rows of one distinct expert for every
// token routed to it, one token at a time (the unit's weights stay in
// registers); h = silu(gate) * up goes to hbuf[(slot0 + token rank) * I + row].
template <int LPR, int PPL, int RG, bool FULL, bool QS, int FMT = kFmtAffine>
__device__ __forceinline__ void gu_compute(const UnionArgs& a, const GuFrag<PPL, RG>& f, uint32_t mask, int slot0,
                                           int row, int li, int KU, const uint4* act, const float* asum,
                                           uint32_t sel) {
#pragma unroll
  for (int p = 0; p < PPL; ++p)
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      touch(f.w[p][r][0]);
      touch(f.w[p][r][1]);
      touch(f.sb[p][r][0]);
      if (!QS && fmt_biased(FMT)) touch(f.sb[p][r][1]);
    }
  uint32_t sbv[PPL][RG][2];
  float nvs[PPL][RG][4];  // nvfp4: decoded scales (gate lo, gate hi, up lo, up hi)
#pragma unroll
  for (int p = 0; p < PPL; ++p)
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      if (FMT == kFmtNvfp4) {
#pragma unroll
        for (int q = 0; q < 4; ++q) nvs[p][r][q] = e4m3_to_f32((f.sb[p][r][0] >> (8 * q)) & 0xFFu);
        sbv[p][r][0] = sbv[p][r][1] = 0u;
      } else if (FMT == kFmtMxfp4 || FMT == kFmtMxfp8) {
        sbv[p][r][0] = f.sb[p][r][0] & 0xFFu;         // E8M0 byte of gate
        sbv[p][r][1] = (f.sb[p][r][0] >> 8) & 0xFFu;  // and of up
      } else if (QS) {
        sbv[p][r][0] = quad_scale_bias<0, 1>(f.sb[p][r][0], sel);
        sbv[p][r][1] = quad_scale_bias<2, 3>(f.sb[p][r][0], sel);
      } else {
        sbv[p][r][0] = f.sb[p][r][0];
        sbv[p][r][1] = f.sb[p][r][1];
      }
    }
  // h of token t for this lane group's RG rows
  auto token_h = [&](int t, float (&h)[RG]) {
    float acc[RG][2];
#pragma unroll
    for (int r = 0; r < RG; ++r) acc[r][0] = acc[r][1] = 0.0f;
#pragma unroll
    for (int p = 0; p < PPL; ++p) {
      const int j = li + LPR * p;
      if (FULL || j < KU) {
        constexpr int NA = fmt_na(FMT);
        const uint4* xa = act + (size_t)t * lds_row_units(8 * NA * KU) + j;
        uint32_t xv[16];
#pragma unroll
        for (int c = 0; c < NA; ++c) {
          const uint4 xc = xa[c * KU];
          xv[4 * c + 0] = xc.x; xv[4 * c + 1] = xc.y; xv[4 * c + 2] = xc.z; xv[4 * c + 3] = xc.w;
        }
        if constexpr (FMT == kFmtMxfp8) {  // 16 inputs per position, natural order
#pragma unroll
          for (int r = 0; r < RG; ++r)
#pragma unroll
            for (int mm = 0; mm < 2; ++mm)
              acc[r][mm] += mx_scaled(dot16_mx8_bf16(opaque<(PPL >= kGuOpaquePpl)>(f.w[p][r][mm]), xv, 0.0f),
                                      sbv[p][r][mm]);
        } else if constexpr (FMT == kFmtAffine8) {  // 16 inputs per position, natural order
          const float xs = asum[(size_t)t * KU + j];
#pragma unroll
          for (int r = 0; r < RG; ++r)
#pragma unroll
            for (int mm = 0; mm < 2; ++mm) {
              const float d = dot16_a8_bf16(opaque<(PPL >= kGuOpaquePpl)>(f.w[p][r][mm]), xv, 0.0f);
              const float sc = bf16_lo_to_f32(sbv[p][r][mm]);
              const float bi = bf16_hi_to_f32(sbv[p][r][mm]) - 2176.0f * sc;
              acc[r][mm] += sc * d + bi * xs;
            }
        } else if constexpr (FMT == kFmtMxfp4) {  // x staged in natural element order
#pragma unroll
          for (int r = 0; r < RG; ++r)
#pragma unroll
            for (int mm = 0; mm < 2; ++mm)
              acc[r][mm] += mx_scaled(dot32_mx_bf16(opaque<(PPL >= kGuOpaquePpl)>(f.w[p][r][mm]), xv, 0.0f),
                                      sbv[p][r][mm]);
        } else if constexpr (FMT == kFmtNvfp4) {
#pragma unroll
          for (int r = 0; r < RG; ++r)
#pragma unroll
            for (int mm = 0; mm < 2; ++mm)
              acc[r][mm] += dot32_nv_bf16(opaque<(PPL >= kGuOpaquePpl)>(f.w[p][r][mm]), xv, nvs[p][r][2 * mm],
                                          nvs[p][r][2 * mm + 1]);
        } else {
          const float xs = asum[(size_t)t * KU + j];
#pragma unroll
          for (int r = 0; r < RG; ++r)
#pragma unroll
            for (int mm = 0; mm < 2; ++mm) {
              const float d = dot32<false>(opaque<(PPL >= kGuOpaquePpl)>(f.w[p][r][mm]), xv, kMagicBytes, 0.0f);
              const float sc = bf16_lo_to_f32(sbv[p][r][mm]);
              const float bi = bf16_hi_to_f32(sbv[p][r][mm]) - 128.0f * sc;
              acc[r][mm] += sc * d + bi * xs;
            }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      // gate total in even lanes, up total in odd lanes, then swapped in
      const float k = reduce_rows<LPR, 2>(acc[r]);
      const float o = dpp_f32<0xB1>(k);
      const float gt = (li & 1) ? o : k, up = (li & 1) ? k : o;
      // silu(g) = g / (1 + e^-g) with the hardware exp and reciprocal (about
      // 1 ulp each, where the IEEE division and libm exp cost ~20
      // instructions per token and row): h's relative error stays near
      // 2^-21, far below its fp16 rounding in the down projection; e^-g
      // overflowing to infinity gives 0, as silu should
      h[r] = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;
    }
  };
  const int ntok = __popc(mask);
  if (ntok <= LPR) {
    // one store per row for all the unit's tokens: lane li stores token
    // min(li, ntok - 1), so the count of stores does not depend on the
    // tokens (the waits on the weight loads in flight stay static)
    const int qsel = min(li, ntok - 1);
    float hsel[RG];
#pragma unroll
    for (int r = 0; r < RG; ++r) hsel[r] = 0.0f;
    uint32_t m = mask;
    for (int c = 0; m; ++c) {
      const int t = __builtin_ctz(m);
      m &= m - 1u;
      float h[RG];
      token_h(t, h);
#pragma unroll
      for (int r = 0; r < RG; ++r) hsel[r] = qsel == c ? h[r] : hsel[r];
    }
#pragma unroll
    for (int r = 0; r < RG; ++r) a.hbuf[(size_t)(slot0 + qsel) * a.I + row + r] = hsel[r];
  } else {  // more tokens than lanes in a group: one store per token and row
    uint32_t m = mask;
    for (int c = 0; m; ++c) {
      const int t = __builtin_ctz(m);
      m &= m - 1u;
      float h[RG];
      token_h(t, h);
#pragma unroll
      for (int r = 0; r < RG; ++r) a.hbuf[(size_t)(slot0 + c) * a.I + row + r] = h[r];
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the loads in flight restart from a known count
  }
}

// Tables for the down and combine kernels (one workgroup; no barriers, so
// each wave writes its share whenever it gets here):
//   hdr[0..2]   status of this call, path, distinct experts u
//   utab[i]     (expert id, token mask, first pair slot, 0) of distinct expert i
//   slot_w[s]   router weight of pair slot s (token t's weights summed over its
//               routes to that expert, ascending route order)
//   slot_dst[s]   output row t * k + c of pair slot s in ys (c = rank of the
//                 slot's expert among token t's distinct experts); tcount[t] = c's
__device__ inline void write_union_tables(const UnionArgs& a, const UnionLds& s, int u, int L, int k) {
  const int tid = threadIdx.x;
  if (tid == 0) {
    const uint32_t st = s.scal[1] ? MOE_Q4_DEV_BAD_ID : 0u;
    a.hdr[0] = a.status_or ? (a.hdr[0] | st) : st;  // status of this call
    a.hdr[1] = MOE_Q4_PATH_UNION;
    a.hdr[2] = (uint32_t)u;
  }
  for (int i = tid; i < u; i += blockDim.x) a.utab[i] = make_int4(s.uniq[i], (int)s.mask[i], s.off[i], 0);
  // one thread per pair slot
  const int npairs = s.off[u];
  for (int sl = tid; sl < npairs; sl += blockDim.x) {
    int lo = 0, hi = u - 1;  // distinct expert owning slot sl: last i with off[i] <= sl
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s.off[mid] <= sl) lo = mid; else hi = mid - 1;
    }
    const int t = nth_set_bit(s.mask[lo], sl - s.off[lo]);
    a.slot_w[sl] = token_expert_weight(s, t, k, s.uniq[lo]);
  }
  for (int t = tid; t < L; t += blockDim.x) {
    int c = 0;
    for (int i = 0; i < u; ++i) {
      const uint32_t m = s.mask[i];
      if ((m >> t) & 1u) a.slot_dst[s.off[i] + __popc(m & ((1u << t) - 1u))] = t * k + c++;
    }
    a.tcount[t] = c;
  }
}

template <int LPR, int PPL, bool FULL, bool QS, int FMT = kFmtAffine, bool MF = false>
__global__ __launch_bounds__(kThreads) void k_gateup(UnionArgs a) {
  constexpr int G = 64 / LPR;           // lane groups per wave
  constexpr int RG = gateup_rows(PPL);
  constexpr int WROWS = G * RG;         // hidden rows of one wave unit
  extern __shared__ __align__(16) unsigned char smem[];
  const int H = a.H, I = a.I, k = a.k, L = a.L, E = a.E;
  const int P = L * k;
  constexpr int NA = fmt_na(FMT);
  const int KU = H / fmt_pos_inputs(FMT), KG = FMT == kFmtAffine32 ? KU : H >> 6;  // positions, affine groups
  uint4* act = reinterpret_cast<uint4*>(smem + a.lds_act);      // [L][NA][KU] bf16 pairs, rows padded
  float* asum = reinterpret_cast<float*>(smem + a.lds_asum);     // [L][KU] sums of each position's inputs
  UnionLds s;
  carve_union(smem + a.lds_union, E, P, s);
  const int tid = threadIdx.x;
  __shared__ int unit_q;  // next dynamically assigned unit of this block
  __shared__ int n_mfma;  // distinct experts on the matrix cores
  if (tid == 0) unit_q = 2 * kWaves;
  stage_routes(a.ids, a.tw, P, s);  // first loads of the kernel
  // stage all tokens' activations (independent of the union; overlaps it):
  // three positions per thread per round, all loads issued first
  {
    constexpr int XB = 3;
    const int nx = L * KU;
    for (int base = tid; base < nx; base += XB * kThreads) {
      uint4 v[XB][NA];
#pragma unroll
      for (int b = 0; b < XB; ++b) {
        const int it = min(base + b * kThreads, nx - 1);
        const int t = it / KU, j = it - t * KU;
        const uint4* xs = reinterpret_cast<const uint4*>(a.x + (size_t)t * H) + NA * j;
#pragma unroll
        for (int c = 0; c < NA; ++c) v[b][c] = xs[c];
      }
#pragma unroll
      for (int b = 0; b < XB; ++b) {
        const int it = base + b * kThreads;
        if (it < nx) {
          const int t = it / KU, j = it - t * KU;
          float sum = 0.0f;
#pragma unroll
          for (int c = 0; c < NA; ++c) {
            if (fmt_biased(FMT)) sum = sum8_bf16(v[b][c], sum);
            // FP4 and 8-bit codes convert to pairs in natural element order
            act[(size_t)t * lds_row_units(H) + c * KU + j] = fmt_natural(FMT) ? v[b][c] : pair_activations(v[b][c]);
          }
          if (fmt_biased(FMT)) asum[(size_t)t * KU + j] = sum;
        }
      }
    }
  }
  build_union(P, k, E, s);  // ends with a barrier
  const int u = s.scal[0];
  // Matrix-core instances: distinct experts with at least kMfmaMinTokens
  // tokens take the matrix cores (16-row tiles, every token at once) when
  // mfma_engaged, the others the GEMV units.  mlist: their indices in
  // ascending order, then the others' at + P.
  int* mlist = reinterpret_cast<int*>(smem + a.lds_mlist);
  int nm = 0;
  if constexpr (MF) {
    static_assert(FMT == kFmtAffine, "matrix-core tiles read 4-bit affine group-64 banks");
    // every wave counts (the same answer), so a call without tiles skips
    // the list and its barrier
    int nmany = 0;
    for (int base = 0; base < u; base += 64) {
      const int i = base + (tid & 63);
      nmany += __popcll(__ballot(i < u && __popc(s.mask[i]) >= kMfmaMinTokens));
    }
    if (mfma_engaged(nmany, u)) {
      if (tid < 64) {
        int cm = 0, cv = 0;
        for (int base = 0; base < u; base += 64) {
          const int i = base + tid;
          const bool many = i < u && __popc(s.mask[i]) >= kMfmaMinTokens;
          const bool few = i < u && !many;
          const unsigned long long bm = __ballot(many), bf = __ballot(few);
          const unsigned long long below = (1ull << tid) - 1ull;
          if (many) mlist[cm + __popcll(bm & below)] = i;
          if (few) mlist[P + cv + __popcll(bf & below)] = i;
          cm += __popcll(bm);
          cv += __popcll(bf);
        }
        if (tid == 0) n_mfma = cm;
      }
      __syncthreads();
      nm = n_mfma;
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
      const int grp = QS ? 2 * (li >> 2) + (LPR / 2) * p
                         : FMT == kFmtAffine32 ? j : FMT == kFmtAffine8 ? (j >> 2) : (j >> 1);
      o.s[p][r] = FMT == kFmtMxfp8 ? (uint32_t)((g * RG + r) * (KU >> 1) + (j >> 1))
                  : fmt_fp4(FMT)   ? (uint32_t)(((g * RG + r) * KU + j) * (FMT == kFmtNvfp4 ? 2 : 1))
                                   : (uint32_t)(((g * RG + r) * KG + grp) * 2);
    }
  // Work units: (distinct expert, WROWS hidden rows).  Block b owns units
  // b, b + nblk, b + 2 nblk, ... (adjacent blocks take adjacent rows, so the
  // chip sweeps each expert's rows in order).  Inside the block the waves
  // take the block's units from an LDS counter: the two waves sharing a SIMD
  // do not progress at the same rate (issue arbitration favours the older
  // one), and a fixed split would leave the younger ones as the kernel's
  // tail.  Each wave streams its units through a ring of three register
  // fragments, two in flight while the third is computed; a unit index past
  // the block's share loads the share's last unit again (cache-resident), so
  // every load is unconditional.
  const int nblk = gridDim.x;
  int b = blockIdx.x;
  if constexpr (MF) {
    if (nm > 0) {
      // the matrix-core tiles first (tile t in block t % nblk); the GEMV
      // units then start at the first block after the tiles, so the blocks
      // that ran a tile take one unit fewer where the units do not divide
      gu_mfma_phase<kWaves>(a, s, mlist, nm, act, asum, reinterpret_cast<float*>(smem + a.lds_red), b, nblk);
      const int ntm = nm * (I / kMfmaRows);
      b = (b + nblk - ntm % nblk) % nblk;
    }
  }
  // GEMV units over the other distinct experts
  auto vexp = [&](int x) { return MF && nm ? mlist[P + x] : x; };
  const int upe = I / WROWS;                // wave units per expert
  const int nunits = (u - nm) * upe;
  const int nub = nunits > b ? (nunits - 1 - b) / nblk + 1 : 0;  // units of this block
  if (wave < nub) {
    auto load = [&](int j, GuFrag<PPL, RG>& f) {
      const int un = b + min(j, nub - 1) * nblk;
      const int x = un / upe, i = vexp(x);
      gu_load<PPL, RG, FULL, QS, FMT>(a, (size_t)wave_uniform(s.uniq[i]) * I + (un - x * upe) * WROWS, WROWS, KU, KG,
                                     li, LPR, lane_sbase, o, f);
    };
    auto compute = [&](int j, const GuFrag<PPL, RG>& f) {
      const int un = b + j * nblk;
      const int x = un / upe, i = vexp(x);
      gu_compute<LPR, PPL, RG, FULL, QS, FMT>(a, f, wave_uniform((int)s.mask[i]), wave_uniform(s.off[i]),
                                         (un - x * upe) * WROWS + g * RG, li, KU, act, asum, sel);
    };
    auto grab = [&]() {
      int v = 0;
      if (lane == 0) v = atomicAdd(&unit_q, 1);
      return __builtin_amdgcn_readfirstlane(v);
    };
    // j0, j1, j2: the units in f0, f1, f2 (increasing: the counter only grows)
    GuFrag<PPL, RG> f0, f1, f2;
    int j0 = wave, j1 = wave + kWaves, j2;
    load(j0, f0);
    load(j1, f1);
    int jn = grab();  // next unit to load, taken one step ahead
    for (;;) {
      j2 = jn; jn = grab();
      load(j2, f2);
      compute(j0, f0);
      if (j1 >= nub) break;
      j0 = jn; jn = grab();
      load(j0, f0);
      compute(j1, f1);
      if (j2 >= nub) break;
      j1 = jn; jn = grab();
      load(j1, f1);
      compute(j2, f2);
      if (j0 >= nub) break;
    }
  }
  // block 0 writes the tables the down and combine kernels read, after its
  // own units so the table work stays off the start of its weight stream
  if (blockIdx.x == 0) write_union_tables(a, s, u, L, k);
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

template <int PPL, int RS, bool FULL, bool QS, int FMT = kFmtAffine>
__device__ __forceinline__ void dn_load(const UnionArgs& a, size_t row0, bool valid, size_t row_fallback, int nrows,
                                        int KU, int KG, int li, int lpr, const unsigned char* lane_sbase,
                                        const DnOffsets<PPL, RS>& o, DnFrag<PPL, RS>& f) {
  if constexpr (fmt_fp4(FMT) || FMT == kFmtMxfp8) {
    // two E4M3 bytes per position (nvfp4), one E8M0 byte per 32 inputs
    // (mxfp4: per position; mxfp8: per two positions)
    constexpr int SB = FMT == kFmtNvfp4 ? 2 : 1;
    const size_t srow = FMT == kFmtNvfp4 ? (size_t)KU * 2 : FMT == kFmtMxfp8 ? (size_t)(KU >> 1) : (size_t)KU;
    const rsrc_t wd = make_rsrc(reinterpret_cast<const unsigned char*>(a.wd) + row0 * KU * 16,
                                valid ? (uint32_t)(nrows * KU * 16) : 0u);
    const rsrc_t ed = make_rsrc(reinterpret_cast<const unsigned char*>(a.sd) + (valid ? row0 : row_fallback) * srow,
                                valid ? (uint32_t)(nrows * srow) : 0u);
#pragma unroll
    for (int r = 0; r < RS; ++r)
#pragma unroll
      for (int p = 0; p < PPL; ++p)
        if (FULL || li + lpr * p < KU) {
          f.w[r][p] = bld16_nt(wd, o.w[r][p]);
          f.sb[r][p] = SB == 2 ? bld2(ed, o.s[r][p]) : bld1(ed, o.s[r][p]);
        }
    (void)KG; (void)lane_sbase;
    return;
  }
  const rsrc_t wd = make_rsrc(reinterpret_cast<const unsigned char*>(a.wd) + row0 * KU * 16,
                              valid ? (uint32_t)(nrows * KU * 16) : 0u);
  const size_t soff = (valid ? row0 : row_fallback) * KG * 2;
  const uint32_t sbb = valid ? (uint32_t)(nrows * KG * 2) : 0u;
#pragma unroll
  for (int r = 0; r < RS; ++r)
#pragma unroll
    for (int p = 0; p < PPL; ++p)
      if (FULL || li + lpr * p < KU) {
        f.w[r][p] = bld16_nt(wd, o.w[r][p]);
        if (QS) {
          if ((r & 1) == 0) f.sb[r][p] = ld4(lane_sbase + soff, o.s[r][p]);
        } else {
          const rsrc_t sd = make_rsrc(reinterpret_cast<const unsigned char*>(a.sd) + row0 * KG * 2, sbb);
          const rsrc_t bd = make_rsrc(reinterpret_cast<const unsigned char*>(a.bd) + row0 * KG * 2, sbb);
          f.sb[r][p] = bld2(sd, o.s[r][p]) | (bld2(bd, o.s[r][p]) << 16);
        }
      }
}

// LDS of a down block: the union table, the work prefix per expert, then
// per staged pair slot its hidden vector as fp16 pairs [NA][KU] (uint4; KU
// positions of 8 NA inputs; plus one pad unit, lds_row_units), the sums of each position's fp16 values [KU],
// the router weight, the slot's ys row and the exponent that undoes the
// slot's power-of-two scaling.
__host__ __device__ constexpr size_t down_slot_bytes(int KU, int na = 4) { return (size_t)KU * (16 * na + 4) + 16 + 12; }
__host__ __device__ constexpr size_t down_lds_base(int P) { return ((size_t)16 * P + 15) & ~size_t(15); }
// bytes before the staged slots: the union table and the work prefix
__host__ __device__ constexpr size_t down_lds_head(int P) {
  return down_lds_base(P) + (((size_t)4 * (P + 1) + 15) & ~size_t(15));
}

// Converts pair slot `slot` (h of one (expert, token) pair, fp32) into staged
// slot `ls`: scaled by the power of two that puts its largest magnitude in
// [2^13, 2^14), rounded to fp16.  The scaling is applied per element as an
// exponent shift (v_ldexp), never as a multiplier 2^n, which would overflow
// for vectors whose entries all lie below 2^-114; sexp gets the inverse
// shift, applied to the slot's outputs.  One wave per slot; a lane converts
// 32 inputs at a time (one position of 4-bit codes, two of 8-bit codes).
// With TWO and `two`, the wave converts slot2 into ls2 as well, both slots'
// loads in flight together (at one position per lane; the 1024-thread
// kernels, at 128 registers a lane, leave TWO off).  KU counts 32-input
// blocks.
template <int NA, bool TWO = false>
__device__ __forceinline__ void down_stage_slot(const UnionArgs& a, int ls, int slot, int KU, uint4* hvs, float* hss,
                                                float* stw, int* sdst, int* sexp, bool natural, bool two = false,
                                                int ls2 = 0, int slot2 = 0) {
  two = TWO && two;
  const int lane = threadIdx.x & 63;
  auto load32 = [&](int sl, int j, float (&v)[32]) {
    const float4* src = reinterpret_cast<const float4*>(a.hbuf + (size_t)sl * a.I + 32 * j);
#pragma unroll
    for (int q4 = 0; q4 < 8; ++q4) {
      const float4 f4 = src[q4];
      v[4 * q4 + 0] = f4.x; v[4 * q4 + 1] = f4.y; v[4 * q4 + 2] = f4.z; v[4 * q4 + 3] = f4.w;
    }
  };
  auto convert = [&](int ls_, int j, const float (&v)[32], int up) {
    float sum = 0.0f;
#pragma unroll
    for (int wi = 0; wi < 4; ++wi) {
      _Float16 hb[8];
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        hb[n] = (_Float16)__builtin_amdgcn_ldexpf(v[8 * wi + n], up);
        sum += (float)hb[n];
      }
      uint4 pk;
      uint32_t* pw = reinterpret_cast<uint32_t*>(&pk);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        // affine codes unpack to (e0,e2),(e4,e6),(e1,e3),(e5,e7); mxfp4 to natural pairs
        const int lo = natural ? 2 * kk : pair_lo(kk), hi = natural ? 2 * kk + 1 : pair_hi(kk);
        pw[kk] = (uint32_t)__builtin_bit_cast(uint16_t, hb[lo]) | ((uint32_t)__builtin_bit_cast(uint16_t, hb[hi]) << 16);
      }
      if constexpr (NA == 4) {
        hvs[(size_t)ls_ * lds_row_units(32 * KU) + wi * KU + j] = pk;
      } else {  // positions 2j and 2j + 1 of 16 inputs, two uint4 each
        hvs[(size_t)ls_ * lds_row_units(32 * KU) + (wi & 1) * (2 * KU) + 2 * j + (wi >> 1)] = pk;
        if (wi & 1) {
          hss[(size_t)ls_ * 2 * KU + 2 * j + (wi >> 1)] = sum;
          sum = 0.0f;
        }
      }
    }
    if constexpr (NA == 4) hss[(size_t)ls_ * KU + j] = sum;
  };
  auto finish = [&](int ls_, int slot_, int ex) {
    if (lane == 0) {
      stw[ls_] = a.slot_w[slot_];
      sdst[ls_] = a.slot_dst[slot_];
      sexp[ls_] = ex - 14;
    }
  };
  // frexp exponent of a wave-wide maximum magnitude (0 for an all-zero vector)
  auto exp_of = [&](float mx) {
    mx = wave_max(mx);
    return mx > 0.0f ? __builtin_amdgcn_frexp_expf(mx) : 0;
  };
  if (KU <= 64) {  // one position per lane: a single pass over registers
    const bool on = lane < KU;
    float v[32], v2[32];
    load32(slot, on ? lane : 0, v);
    if (two) load32(slot2, on ? lane : 0, v2);
    float mx = 0.0f;
#pragma unroll
    for (int n = 0; n < 32; ++n) mx = fmaxf(mx, on ? fabsf(v[n]) : 0.0f);
    const int ex = exp_of(mx);
    if (on) convert(ls, lane, v, 14 - ex);
    finish(ls, slot, ex);
    if (two) {
      float mx2 = 0.0f;
#pragma unroll
      for (int n = 0; n < 32; ++n) mx2 = fmaxf(mx2, on ? fabsf(v2[n]) : 0.0f);
      const int ex2 = exp_of(mx2);
      if (on) convert(ls2, lane, v2, 14 - ex2);
      finish(ls2, slot2, ex2);
    }
    return;
  }
  // several positions per lane: the maximum first, then a second read
  for (int q = 0; q < (two ? 2 : 1); ++q) {
    const int sl = q ? slot2 : slot, ls_ = q ? ls2 : ls;
    float mx = 0.0f;
    for (int j = lane; j < KU; j += 64) {
      float v[32];
      load32(sl, j, v);
#pragma unroll
      for (int n = 0; n < 32; ++n) mx = fmaxf(mx, fabsf(v[n]));
    }
    const int ex = exp_of(mx);
    for (int j = lane; j < KU; j += 64) {
      float v[32];
      load32(sl, j, v);
      convert(ls_, j, v, 14 - ex);
    }
    finish(ls_, sl, ex);
  }
}

// One step: RS rows of this lane group against NT converted hidden vectors;
// each token's RS row totals, times its router weight and shifted back by
// the exponent of its hidden vector's scaling, go to its ys row in one store
// (every lane stores its residue's row; token slots past the expert's count
// write to the sink).
template <int LPR, int PPL, int RS, int NT, bool FULL, bool QS, int FMT = kFmtAffine>
__device__ __forceinline__ void dn_step(const UnionArgs& a, const DnFrag<PPL, RS>& f, const uint32_t (&hv)[NT][PPL][16],
                                       const float (&hs)[NT][PPL], const float (&tw)[NT], const int (&te)[NT],
                                       float* const (&dst)[NT], int row0, int li, int KU, uint32_t sel) {
#pragma unroll
  for (int r = 0; r < RS; ++r)
#pragma unroll
    for (int p = 0; p < PPL; ++p) {
      touch(f.w[r][p]);
      if (fmt_fp4(FMT) || !QS || (r & 1) == 0) touch(f.sb[r][p]);
    }
  float acc[NT][RS];
#pragma unroll
  for (int c = 0; c < NT; ++c)
#pragma unroll
    for (int r = 0; r < RS; ++r) acc[c][r] = 0.0f;
#pragma unroll
  for (int r = 0; r < RS; ++r) {
#pragma unroll
    for (int p = 0; p < PPL; ++p) {
      if (FULL || li + LPR * p < KU) {
        if constexpr (FMT == kFmtMxfp8) {  // 16 inputs per position, natural order
#pragma unroll
          for (int c = 0; c < NT; ++c) acc[c][r] += mx_scaled(dot16_mx8_f16(f.w[r][p], hv[c][p], 0.0f), f.sb[r][p]);
        } else if constexpr (FMT == kFmtAffine8) {
          const float sc = bf16_lo_to_f32(f.sb[r][p]);
          const float bi = bf16_hi_to_f32(f.sb[r][p]) - 1024.0f * sc;
#pragma unroll
          for (int c = 0; c < NT; ++c) acc[c][r] += sc * dot16_a8_f16(f.w[r][p], hv[c][p], 0.0f) + bi * hs[c][p];
        } else if constexpr (FMT == kFmtMxfp4) {  // hidden vectors staged as fp16 pairs in natural order
#pragma unroll
          for (int c = 0; c < NT; ++c) acc[c][r] += mx_scaled(dot32_mx_f16(f.w[r][p], hv[c][p], 0.0f), f.sb[r][p]);
        } else if constexpr (FMT == kFmtNvfp4) {
          const float s0 = e4m3_to_f32(f.sb[r][p] & 0xFFu), s1 = e4m3_to_f32((f.sb[r][p] >> 8) & 0xFFu);
#pragma unroll
          for (int c = 0; c < NT; ++c) acc[c][r] += dot32_nv_f16(f.w[r][p], hv[c][p], s0, s1);
        } else {
          uint32_t sb;
          if (QS)
            sb = (r & 1) ? quad_scale_bias<2, 3>(f.sb[r & ~1][p], sel) : quad_scale_bias<0, 1>(f.sb[r][p], sel);
          else
            sb = f.sb[r][p];
          const float sc = bf16_lo_to_f32(sb);
          const float bi = bf16_hi_to_f32(sb) - 1024.0f * sc;
#pragma unroll
          for (int c = 0; c < NT; ++c) {
            const float d = dot32<true>(f.w[r][p], hv[c][p], kMagicBytesF16, 0.0f);
            acc[c][r] += sc * d + bi * hs[c][p];
          }
        }
      }
    }
  }
  const int rr = li & (RS - 1);
#pragma unroll
  for (int c = 0; c < NT; ++c) dst[c][row0 + rr] = __builtin_amdgcn_ldexpf(tw[c] * reduce_rows<LPR, RS>(acc[c]), te[c]);
}

// One (expert, token chunk) segment of a down wave: read the chunk's
// converted hidden vectors from LDS, then stream the unit's row steps gj ..
// gj + klast through a ring of three register fragments (two in flight).
template <int LPR, int PPL, bool FULL, bool QS, int NT, int RS, int WSTEP, int FMT = kFmtAffine>
__device__ __forceinline__ void dn_segment(const UnionArgs& a, size_t ebase, int ls0, int nt, int gj, int klast,
                                           int li, int g, int KU, int KG, int H, const unsigned char* lane_sbase,
                                           const DnOffsets<PPL, RS>& o, uint32_t sel, const uint4* hvs,
                                           const float* hss, const float* stw, const int* sdst, const int* sexp,
                                           float* rows_dst = nullptr) {
  // prefetches past the last step are zero-range no-ops
  auto load = [&](int kk, DnFrag<PPL, RS>& fr) {
    const bool valid = kk <= klast;
    const size_t row0 = ebase + (size_t)(gj + min(kk, klast)) * WSTEP;
    dn_load<PPL, RS, FULL, QS, FMT>(a, row0, valid, row0, WSTEP, KU, KG, li, LPR, lane_sbase, o, fr);
  };
  DnFrag<PPL, RS> f0, f1, f2;
  load(0, f0);
  load(1, f1);

  uint32_t hv[NT][PPL][16];
  float hs[NT][PPL], tw[NT];
  int te[NT];
  float* dst[NT];
#pragma unroll
  for (int c = 0; c < NT; ++c) {
    const bool live = c < nt;
    const int ls = ls0 + (live ? c : 0);
#pragma unroll
    for (int p = 0; p < PPL; ++p) {
      const int j = li + LPR * p;
      if (FULL || j < KU) {
        constexpr int NA = fmt_na(FMT);
        const uint4* hp = hvs + (size_t)ls * lds_row_units(8 * NA * KU) + j;
#pragma unroll
        for (int wi = 0; wi < NA; ++wi) {
          const uint4 h4 = hp[wi * KU];
          hv[c][p][4 * wi + 0] = h4.x; hv[c][p][4 * wi + 1] = h4.y;
          hv[c][p][4 * wi + 2] = h4.z; hv[c][p][4 * wi + 3] = h4.w;
        }
        hs[c][p] = hss[(size_t)ls * KU + j];
      } else {
#pragma unroll
        for (int n = 0; n < 16; ++n) hv[c][p][n] = 0u;
        hs[c][p] = 0.0f;
      }
    }
    tw[c] = live ? stw[ls] : 0.0f;
    te[c] = live ? sexp[ls] : 0;
    dst[c] = live ? a.ys + (size_t)wave_uniform(sdst[ls]) * H : a.ys_dummy;
    if (rows_dst) dst[c] = rows_dst;  // one token: the block's row slice in LDS
  }

  auto step = [&](int kk, const DnFrag<PPL, RS>& fr) {
    dn_step<LPR, PPL, RS, NT, FULL, QS, FMT>(a, fr, hv, hs, tw, te, dst, (gj + kk) * WSTEP + g * RS, li, KU, sel);
  };
#pragma unroll 1
  for (int kk = 0;; kk += 3) {
    load(kk + 2, f2);
    step(kk, f0);
    if (kk + 1 > klast) break;
    load(kk + 3, f0);
    step(kk + 1, f1);
    if (kk + 2 > klast) break;
    load(kk + 4, f1);
    step(kk + 2, f2);
    if (kk + 3 > klast) break;
  }
}

// threads of a down block: one block per CU, as many waves as the registers
// allow (the waves of a CU share the converted hidden vectors and one LDS
// work counter); 1024 (at most 128 registers a lane) only for one token per
// pass and one position per lane, where the ring fits in them
__host__ __device__ constexpr int down_threads(int nt, int ppl) { return nt == 1 && ppl == 1 ? 1024 : 512; }
constexpr int kDownUnitSteps = 4;  // row steps per down work unit

// Down projection and router weighting of every (distinct expert, token)
// pair.  Work units: (distinct expert, kDownUnitSteps row steps), numbered
// expert-major; block b takes a contiguous range of them, so it touches one
// or two experts and converts only their tokens' hidden vectors (into LDS,
// once).  Its waves take the units from an LDS counter (the first unit of
// each wave fixed), so waves that get fewer issue slots do less of the
// block's share.  A unit runs every token of its expert, NT at a time.
template <int LPR, int PPL, bool FULL, bool QS, int NT, int FMT = kFmtAffine, bool MF = false>
__global__ __launch_bounds__(down_threads(NT, PPL)) void k_down(UnionArgs a) {
  constexpr int G = 64 / LPR;
  constexpr int RS = down_rows(G);  // a wave step covers G * RS rows
  constexpr int WSTEP = G * RS;
  constexpr int NW = down_threads(NT, PPL) / 64;
  static_assert(!QS || RS % 2 == 0, "quad-shared scales pair rows");
  extern __shared__ __align__(16) unsigned char smem[];
  const int H = a.H, I = a.I, P = a.L * a.k;
  constexpr int NA = fmt_na(FMT);
  const int KU = I / fmt_pos_inputs(FMT), KG = FMT == kFmtAffine32 ? KU : I >> 6;  // positions, affine groups
  const int SM = a.dn_slots;  // pair slots converted at a time
  int4* utab = reinterpret_cast<int4*>(smem);
  int* wpre = reinterpret_cast<int*>(smem + down_lds_base(P));     // [P + 1] work prefix per expert
  uint4* hvs = reinterpret_cast<uint4*>(smem + down_lds_head(P));  // [SM][NA][KU], rows padded
  float* hss = reinterpret_cast<float*>(hvs + (size_t)SM * lds_row_units(I));  // [SM][KU]
  float* stw = hss + (size_t)SM * KU;                                 // [SM]
  int* sdst = reinterpret_cast<int*>(stw + SM);                       // [SM]
  int* sexp = sdst + SM;                                              // [SM]
  __shared__ int unit_q;  // next dynamically assigned unit (block-relative)
  const int tid = threadIdx.x;
  const int umax = min(P, a.E);
  const int u = min((int)a.hdr[2], umax);
  const int spe = H / WSTEP;  // row steps per expert
  const int nrb = (spe + kDownUnitSteps - 1) / kDownUnitSteps;  // units per expert
  // Work of a unit: its token chunks (each streams the unit's rows once).
  // wpre[i] = work of the units of experts before i (wave 0, straight from
  // the table in memory); blocks take equal shares of the total, each share
  // a contiguous range of units.
  // A unit's work counts its token chunks (weight 4 each: each streams the
  // unit's rows) plus its tokens (weight 1 each: the products per token),
  // so a chunk of NT tokens weighs more than a chunk of one (measured: the
  // blocks holding two-token experts had set the kernel's tail at L = 8).
  // With one token every unit is one single-token chunk and the shares are
  // plain unit counts.
  const bool uniform = a.L == 1;
  // Matrix-core instances: experts with at least kMfmaMinTokens tokens run
  // 16-row tiles, every token of the pass at once, when mfma_engaged (the
  // same rule as the gate/up kernel's); a unit of theirs streams its rows
  // once, so it weighs one chunk plus an eighth per token.
  static_assert(!MF || (FMT == kFmtAffine && down_threads(NT, PPL) == 512),
                "matrix-core tiles: 4-bit affine banks, 512-thread blocks");
  __shared__ int mf_min;  // tokens from which an expert runs as tiles
  if (tid < 64 && !uniform) {
    int nmany = 0;
    if (MF)
      for (int base = 0; base < u; base += 64) {
        const int i = base + tid;
        nmany += __popcll(__ballot(i < u && __popc((uint32_t)a.utab[i].y) >= kMfmaMinTokens));
      }
    const int mmin = MF && mfma_engaged(nmany, u) ? kMfmaMinTokens : 33;
    if (tid == 0) mf_min = mmin;
    int carry = 0;
    for (int base = 0; base < u; base += 64) {
      const int i = base + tid;
      const int n = i < u ? __popc((uint32_t)a.utab[i].y) : 0;
      const int w = i >= u        ? 0
                    : n >= mmin ? nrb * (4 + (n + 7) / 8)
                                : nrb * (4 * ((n + NT - 1) / NT) + n);
      const int incl = wave_incl_scan(w);
      if (i < u) wpre[i] = carry + incl - w;
      carry += __shfl(incl, 63, 64);
    }
    if (tid == 0) wpre[u] = carry;
  }
  for (int i = tid; i < umax; i += blockDim.x) utab[i] = a.utab[i];
  if (tid == 0) {
    unit_q = NW;
    if (uniform) mf_min = 33;
  }
  __syncthreads();
  const int tile_min = mf_min;
  const int nblk = gridDim.x, b = blockIdx.x;
  const int lane = tid & 63;
  const int wave = wave_uniform(tid >> 6);
  auto grab = [&]() {
    int v = 0;
    if (lane == 0) v = atomicAdd(&unit_q, 1);
    return __builtin_amdgcn_readfirstlane(v);
  };
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
      const int grp = QS ? 2 * (li >> 2) + (LPR / 2) * p
                         : FMT == kFmtAffine32 ? j : FMT == kFmtAffine8 ? (j >> 2) : (j >> 1);
      o.s[r][p] = FMT == kFmtMxfp8 ? (uint32_t)((g * RS + r) * (KU >> 1) + (j >> 1))
                  : fmt_fp4(FMT)   ? (uint32_t)(((g * RS + r) * KU + j) * (FMT == kFmtNvfp4 ? 2 : 1))
                                   : (uint32_t)(((g * RS + srow) * KG + grp) * 2);
    }

  if (NT == 1 && a.dn_rows) {
    // One token (so one pair slot per distinct expert, slot i of expert i):
    // block b owns row steps [s0, s1) of every expert, stages all u hidden
    // vectors, runs units (expert, chunk of its steps) into a row slice per
    // expert in LDS, then adds the slices in ascending expert order -- the
    // combine kernel's order -- and writes out itself.
    const int s0 = (int)((long long)spe * b / nblk), s1 = (int)((long long)spe * (b + 1) / nblk);
    const int ns = s1 - s0, nrows = ns * WSTEP;
    if (ns <= 0) return;  // uniform over the block
    float* part = reinterpret_cast<float*>(sexp + SM);  // [u][nrows]
    for (int sl = wave; sl < u; sl += 2 * NW)  // this wave's slots two at a time
      down_stage_slot<NA, (NW < 16)>(a, sl, sl, I >> 5, hvs, hss, stw, sdst, sexp, fmt_natural(FMT), sl + NW < u,
                                     sl + NW, sl + NW);
    __syncthreads();
    const int nch = max(1, min(ns, NW / max(u, 1)));  // step chunks per expert
    const int cs = (ns + nch - 1) / nch;
    for (int j = wave; j < u * nch; j = grab()) {
      const int i = j / nch, g0 = (j - i * nch) * cs, g1 = min(ns, g0 + cs);
      if (g0 >= g1) continue;
      const size_t ebase = (size_t)wave_uniform(utab[i].x) * H + (size_t)s0 * WSTEP;
      dn_segment<LPR, PPL, FULL, QS, 1, RS, WSTEP, FMT>(a, ebase, i, 1, g0, g1 - g0 - 1, li, g, KU, KG, H, lane_sbase,
                                                       o, sel, hvs, hss, stw, sdst, sexp, part + (size_t)i * nrows);
    }
    __syncthreads();
    for (int r = tid; r < nrows; r += blockDim.x) {
      float acc = 0.0f;
      for (int i = 0; i < u; ++i) acc += part[i * nrows + r];
      const size_t m = (size_t)s0 * WSTEP + r;
      if (a.out_f32)
        reinterpret_cast<float*>(a.out)[m] = acc;
      else
        reinterpret_cast<uint16_t*>(a.out)[m] = (uint16_t)f32_to_bf16_rne(acc);
    }
    return;
  }

  const int wtot = uniform ? u * nrb : wpre[u];
  // first unit whose work starts at or after offset x
  auto unit_at = [&](long long x) {
    if (x >= wtot) return u * nrb;
    if (uniform) return (int)x;
    int lo = 0, hi = u - 1;  // last expert i with wpre[i] <= x
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (wpre[mid] <= x) lo = mid; else hi = mid - 1;
    }
    const int nch = (wpre[lo + 1] - wpre[lo]) / nrb;
    return lo * nrb + (int)((x - wpre[lo] + nch - 1) / nch);
  };
  const int ub = unit_at((long long)wtot * b / nblk);
  const int nub = unit_at((long long)wtot * (b + 1) / nblk) - ub;  // units of this block
  if (nub <= 0) return;  // uniform over the block
  const int s_lo = utab[ub / nrb].z;
  const int4 ehi = utab[(ub + nub - 1) / nrb];
  const int s_hi = ehi.z + __popc((uint32_t)ehi.y);  // pair slots of the block's experts

  // Usually one pass; more when the block's experts have more pair slots
  // than the LDS holds (each pass runs the block's units for its slots).
  for (int c0 = s_lo; c0 < s_hi; c0 += SM) {
    const int c1 = min(s_hi, c0 + SM);
    if (tid == 0) unit_q = NW;
    for (int sl = c0 + wave; sl < c1; sl += 2 * NW)  // this wave's slots two at a time
      down_stage_slot<NA, (NW < 16)>(a, sl - c0, sl, I >> 5, hvs, hss, stw, sdst, sexp, fmt_natural(FMT),
                                     sl + NW < c1, sl + NW - c0, sl + NW);
    __syncthreads();
    if constexpr (MF) {
      // Matrix-core instances: the tiles of the block's matrix-core units
      // first (task j: 16-row tile j % TPU of unit ub + j / TPU; wave w
      // takes tasks w, w + NW, ..., all through one ring), then the GEMV
      // units from the counter.
      constexpr int TPU = kDownUnitSteps * WSTEP / kMfmaRows;
      static_assert((kDownUnitSteps * WSTEP) % kMfmaRows == 0, "whole tiles per unit");
      auto mtile = [&](int j, DnTile& t) {
        const int un = ub + j / TPU, sub = j % TPU;
        const int i = un / nrb, rb = un - i * nrb;
        const int4 ent = utab[i];
        const int n = __popc((uint32_t)wave_uniform(ent.y)), off = wave_uniform(ent.z);
        const int gj = rb * kDownUnitSteps, rows = min(kDownUnitSteps, spe - gj) * WSTEP;
        const int t_lo = max(off, c0), t_hi = min(off + n, c1);
        if (n < tile_min || sub * kMfmaRows >= rows || t_hi <= t_lo) return false;
        t.e = wave_uniform(ent.x);
        t.r0 = gj * WSTEP + sub * kMfmaRows;
        t.ls0 = t_lo - c0;
        t.n = t_hi - t_lo;
        return true;
      };
      if (tile_min <= 32) dn_mfma_run(a, mtile, wave, NW, nub * TPU, hvs, hss, stw, sdst, sexp);
    }
    // GEMV tasks: (unit, chunk of NT tokens), cpu chunks a unit -- the most
    // any of the block's experts has in this pass (units with fewer skip the
    // rest).  The chunks of one unit are consecutive tasks, so the waves run
    // them side by side (the re-read rows hit the caches) instead of one
    // wave running them in turn, which had left the waves holding experts
    // with many tokens as the block's tail.
    int cpu = 1;
    for (int i = ub / nrb; i <= (ub + nub - 1) / nrb; ++i) {
      const int4 ent = utab[i];
      const int n = __popc((uint32_t)ent.y);
      if (!(MF && n >= tile_min)) cpu = max(cpu, (min(ent.z + n, c1) - max(ent.z, c0) + NT - 1) / NT);
    }
    for (int j = wave; j < nub * cpu; j = grab()) {
      const int jd = j / cpu;
      const int un = ub + jd, ch = j - jd * cpu;
      const int i = un / nrb, rb = un - i * nrb;
      const int4 ent = utab[i];
      const int e = wave_uniform(ent.x), off = wave_uniform(ent.z), n = __popc((uint32_t)wave_uniform(ent.y));
      if (MF && n >= tile_min) continue;  // ran as tiles
      const int t0 = max(off, c0) + ch * NT, t_hi = min(off + n, c1);
      if (t0 >= t_hi) continue;
      const int nt = min(NT, t_hi - t0);
      const size_t ebase = (size_t)e * H;
      const int gj = rb * kDownUnitSteps;
      const int klast = min(kDownUnitSteps, spe - gj) - 1;
      if (NT > 1 && nt == 1)
        dn_segment<LPR, PPL, FULL, QS, 1, RS, WSTEP, FMT>(a, ebase, t0 - c0, 1, gj, klast, li, g, KU, KG, H,
                                                         lane_sbase, o, sel, hvs, hss, stw, sdst, sexp);
      else
        dn_segment<LPR, PPL, FULL, QS, NT, RS, WSTEP, FMT>(a, ebase, t0 - c0, nt, gj, klast, li, g, KU, KG, H,
                                                          lane_sbase, o, sel, hvs, hss, stw, sdst, sexp);
    }
    __syncthreads();  // the converted slots and the counter are reused
  }
}

}  // namespace moeq4
