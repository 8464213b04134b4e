// Union path of the SwitchGLU-q4 MoE layer for gfx950 (MI355X).
//
// Three kernels:
//   k_route_union   the distinct experts of the L*k routes, their token masks,
//                   summed router weights and the slot -> distinct-id map
//                   (exported on its own for bit-exact checks);
//   k_gateup        for each distinct expert and block of 32 hidden rows: the
//                   gate and up dequant-GEMVs of every token routed to that
//                   expert, fused in one pass over the packed weights, then
//                   h = silu(gate) * up kept in fp32 (written as an exact
//                   bf16 hi + lo pair) with its per-32-row sum;
//   k_down          for each distinct expert and block of 32 output rows: the
//                   down dequant-GEMV of the expert's hidden vectors times the
//                   tokens' router weights, written per (expert, token); the
//                   last work item of a row block adds the experts' parts in
//                   ascending expert order (deterministic, no float atomics).
//
// Sources (web pages): streaming every distinct routed expert once and
// applying it to each position routed to it is the union gather of the mlx
// discussion "Small-L fused expert gather for fine-grained MoE decode"
// (implication 1 of the overlap section); running gate and up in one pass with
// SiLU applied to the gate before the product follows the splash PR "perf:
// Apple7/8 MoE gate and up in one decode pass" (section "What changed") and the
// SwitchGLU order of the mlx issue "gather_qmm at M=1 streams 4-bit expert
// weights at ~half the bandwidth of M=4" (moe_bench script).
//
// Inner product with affine codes.  For 32 consecutive inputs c of one row
// (one 16-byte load, one (scale s, bias b) group half):
//     sum_c a_c (s q_c + b) = s * D + (b - 128 s) * A,
//     D = sum_c a_c (128 + q_c),  A = sum_c a_c,
// where 128 + q_c is built exactly as bf16 by OR-ing the nibble into the
// mantissa of 128.0 and D accumulates with bf16 dot2 in fp32.  A is computed
// once per activation position and stored beside the activations.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_q4.h"
#include "moe_q4_device.h"
#include "moe_q4_internal.h"

namespace moeq4 {

// Lane layout of one work item (32 rows of one expert).  A row of K inputs is
// K/32 16-byte positions; LPR lanes (a power of two <= 64) split them, lane li
// taking positions li, li + LPR, ...  A wave holds 64/LPR lane groups; each
// group computes RPG rows.
template <int LPR>
struct Tile {
  static constexpr int G = 64 / LPR;
  static constexpr int RPG = LPR >= 32 ? LPR / 16 : 1;
  static constexpr int RPW = G * RPG;
  static constexpr int NW = kRows / RPW;
  static constexpr int NTHR = 64 * NW;
  static_assert(NW >= 1 && NW * RPW == kRows, "tile shape");
};

// Accumulates, for the RPG rows of this lane group and NMAT matrices, the
// partial inner products over this lane's positions with NT staged activation
// vectors.  act: LDS planes [NT][NCH][KU] of uint4 (NCH = 4: bf16 pairs of one
// vector; NCH = 8: bf16 hi pairs then lo pairs of an fp32 vector); asum: LDS
// [NT][KU] per-position sums of the activations.
template <int LPR, int PPL, int NT, int NMAT, int NCH>
__device__ __forceinline__ void rows_dot(const uint4* const (&W)[NMAT], const uint16_t* const (&S)[NMAT],
                                         const uint16_t* const (&B)[NMAT], int KU, int KG, const uint4* act,
                                         const float* asum, int nt, int li, float (&acc)[NT][Tile<LPR>::RPG][NMAT]) {
  constexpr int RPG = Tile<LPR>::RPG;
#pragma unroll
  for (int p = 0; p < PPL; ++p) {
    const int j = li + LPR * p;
    if (j >= KU) continue;
    uint4 w[NMAT][RPG];
    uint16_t sv[NMAT][RPG], bv[NMAT][RPG];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int r = 0; r < RPG; ++r) {
        w[m][r] = W[m][(size_t)r * KU + j];
        sv[m][r] = S[m][(size_t)r * KG + (j >> 1)];
        bv[m][r] = B[m][(size_t)r * KG + (j >> 1)];
      }
    uint32_t a[NT][NCH * 4];
    float as[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t < nt) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          const uint4 v = act[((size_t)t * NCH + c) * KU + j];
          a[t][4 * c + 0] = v.x;
          a[t][4 * c + 1] = v.y;
          a[t][4 * c + 2] = v.z;
          a[t][4 * c + 3] = v.w;
        }
        as[t] = asum[(size_t)t * KU + j];
      }
    }
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int r = 0; r < RPG; ++r) {
        uint32_t q[16];
        unpack_word(w[m][r].x, q + 0);
        unpack_word(w[m][r].y, q + 4);
        unpack_word(w[m][r].z, q + 8);
        unpack_word(w[m][r].w, q + 12);
        const float s = bf16_to_f32(sv[m][r]);
        const float b = bf16_to_f32(bv[m][r]) - 128.0f * s;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if (t < nt) {
            float d = 0.0f;
#pragma unroll
            for (int c = 0; c < NCH; ++c)
#pragma unroll
              for (int kk = 0; kk < 4; ++kk) d = dot2_bf16(q[(c & 3) * 4 + kk], a[t][4 * c + kk], d);
            acc[t][r][m] += s * d + b * as[t];
          }
        }
      }
  }
}

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
  const int EW = (E + 31) >> 5;
  UnionLds s;
  s.bitmap = reinterpret_cast<uint32_t*>(smem);
  s.scan = reinterpret_cast<int32_t*>(s.bitmap + EW);
  s.uniq = s.scan + EW;
  s.mask = reinterpret_cast<uint32_t*>(s.uniq + P);
  s.off = reinterpret_cast<int32_t*>(s.mask + P);
  s.scal = s.off + P + 1;
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

template <int LPR, int PPL, int NT>
__global__ __launch_bounds__(Tile<LPR>::NTHR) void k_gateup(UnionArgs a) {
  using T = Tile<LPR>;
  constexpr int RPG = T::RPG;
  extern __shared__ __align__(16) unsigned char smem[];
  const int H = a.H, I = a.I, k = a.k, L = a.L, E = a.E;
  const int P = L * k;
  const int KU = H >> 5;          // 16-byte positions per gate/up row
  const int KG = H >> 6;          // scale groups per gate/up row
  const int KUd = I >> 5;         // 16-byte positions per down row (= row blocks of I)
  const int NRB = I / kRows;

  uint4* act = reinterpret_cast<uint4*>(smem + a.lds_act);
  float* asum = reinterpret_cast<float*>(smem + a.lds_asum);
  uint32_t* hpair = reinterpret_cast<uint32_t*>(smem + a.lds_hpair);   // [NT][32] bf16 hi | lo << 16
  float* hval = reinterpret_cast<float*>(smem + a.lds_hval);           // [NT][32] hi + lo
  int32_t* toks = reinterpret_cast<int32_t*>(smem + a.lds_toks);       // [32]
  UnionLds s;
  const int EW = (E + 31) >> 5;
  s.bitmap = reinterpret_cast<uint32_t*>(smem + a.lds_union);
  s.scan = reinterpret_cast<int32_t*>(s.bitmap + EW);
  s.uniq = s.scan + EW;
  s.mask = reinterpret_cast<uint32_t*>(s.uniq + P);
  s.off = reinterpret_cast<int32_t*>(s.mask + P);
  s.scal = s.off + P + 1;

  build_union(a.ids, P, k, E, s);
  const int u = s.scal[0];
  const int tid = threadIdx.x;
  if (blockIdx.x == 0) {
    for (int i = tid; i < (H / kRows); i += blockDim.x) a.cnt[i] = 0u;  // down-combine counters
    if (tid == 0) {
      a.hdr[0] = s.scal[1] ? MOE_Q4_DEV_BAD_ID : 0u;  // status of this call
      a.hdr[1] = MOE_Q4_PATH_UNION;
      a.hdr[2] = (uint32_t)u;
    }
  }

  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane / LPR, li = lane % LPR;
  const int row_in_item = wave * T::RPW + g * RPG;  // first of this group's RPG rows

  for (int item = blockIdx.x; item < u * NRB; item += gridDim.x) {
    const int i = item / NRB, rb = item - i * NRB;
    const int e = s.uniq[i];
    const uint32_t mask = s.mask[i];
    const int ntok = __popc(mask);
    const int slot0 = s.off[i];
    const size_t row0 = (size_t)e * I + (size_t)rb * kRows + row_in_item;
    const uint4* W[2] = {reinterpret_cast<const uint4*>(a.wg) + row0 * KU,
                         reinterpret_cast<const uint4*>(a.wu) + row0 * KU};
    const uint16_t* S[2] = {a.sg + row0 * KG, a.su + row0 * KG};
    const uint16_t* B[2] = {a.bg + row0 * KG, a.bu + row0 * KG};

    for (int t0 = 0; t0 < ntok; t0 += NT) {
      const int nt = __builtin_amdgcn_readfirstlane(min(NT, ntok - t0));
      __syncthreads();  // previous chunk's readers of act / hpair are done
      if (tid < 32) toks[tid] = (tid < nt) ? nth_set_bit(mask, t0 + tid) : 0;
      __syncthreads();
      // stage the chunk's activations: bf16 pairs in code order + 32-element sums
      for (int it = tid; it < nt * KU; it += blockDim.x) {
        const int t = it / KU, j = it - t * KU;
        const uint4* xs = reinterpret_cast<const uint4*>(a.x + (size_t)toks[t] * H) + 4 * j;
        float sum = 0.0f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint4 v = xs[c];
          sum = sum8_bf16(v, sum);
          act[((size_t)t * 4 + c) * KU + j] = pair_activations(v);
        }
        asum[(size_t)t * KU + j] = sum;
      }
      __syncthreads();

      float acc[NT][RPG][2];
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < RPG; ++r) acc[t][r][0] = acc[t][r][1] = 0.0f;
      rows_dot<LPR, PPL, NT, 2, 4>(W, S, B, KU, KG, act, asum, nt, li, acc);

#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < RPG; ++r) {
          const float gs = group_sum<LPR>(acc[t][r][0]);
          const float us = group_sum<LPR>(acc[t][r][1]);
          if (li == 0 && t < nt) {
            const float h = gs / (1.0f + expf(-gs)) * us;
            const uint32_t hi = f32_to_bf16_rne(h);
            const float hif = __uint_as_float(hi << 16);
            const uint32_t lo = f32_to_bf16_rne(h - hif);
            hpair[t * kRows + row_in_item + r] = hi | (lo << 16);
            hval[t * kRows + row_in_item + r] = hif + __uint_as_float(lo << 16);
          }
        }
      __syncthreads();
      // hidden vectors of the chunk -> workspace, in the down kernel's pair order
      for (int it = tid; it < nt * 32; it += blockDim.x) {
        const int t = it >> 5, q = it & 31;
        const int half = q >> 4, qq = q & 15;           // half 0: hi pairs, 1: lo pairs
        const int n0 = 8 * (qq >> 2) + (qq & 3), n1 = n0 + 4;
        const uint32_t p0 = hpair[t * kRows + n0], p1 = hpair[t * kRows + n1];
        const uint32_t v = half ? ((p0 >> 16) | (p1 & 0xFFFF0000u)) : ((p0 & 0xFFFFu) | (p1 << 16));
        a.hbuf[((size_t)(slot0 + t0 + t) * KUd + rb) * 32 + q] = v;
      }
      if (tid < nt) {
        float sum = 0.0f;
        for (int n = 0; n < kRows; ++n) sum += hval[tid * kRows + n];
        a.hsum[(size_t)(slot0 + t0 + tid) * KUd + rb] = sum;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// down + router-weighted combine
// ---------------------------------------------------------------------------

template <int LPR, int PPL, int NT>
__global__ __launch_bounds__(Tile<LPR>::NTHR) void k_down(UnionArgs a) {
  using T = Tile<LPR>;
  constexpr int RPG = T::RPG;
  extern __shared__ __align__(16) unsigned char smem[];
  const int H = a.H, I = a.I, k = a.k, L = a.L, E = a.E;
  const int P = L * k;
  const int KU = I >> 5;   // 16-byte positions per down row
  const int KG = I >> 6;
  const int NRB = H / kRows;

  uint4* act = reinterpret_cast<uint4*>(smem + a.lds_act);
  float* asum = reinterpret_cast<float*>(smem + a.lds_asum);
  int32_t* toks = reinterpret_cast<int32_t*>(smem + a.lds_toks);   // [32]
  float* tokw = reinterpret_cast<float*>(smem + a.lds_tokw);       // [32]
  int32_t* last = reinterpret_cast<int32_t*>(smem + a.lds_flag);
  UnionLds s;
  const int EW = (E + 31) >> 5;
  s.bitmap = reinterpret_cast<uint32_t*>(smem + a.lds_union);
  s.scan = reinterpret_cast<int32_t*>(s.bitmap + EW);
  s.uniq = s.scan + EW;
  s.mask = reinterpret_cast<uint32_t*>(s.uniq + P);
  s.off = reinterpret_cast<int32_t*>(s.mask + P);
  s.scal = s.off + P + 1;

  build_union(a.ids, P, k, E, s);
  const int u = s.scal[0];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane / LPR, li = lane % LPR;
  const int row_in_item = wave * T::RPW + g * RPG;

  if (u == 0) {  // no valid route at all: the layer output is zero
    for (int it = blockIdx.x * blockDim.x + tid; it < L * H; it += gridDim.x * blockDim.x) {
      if (a.out_f32)
        reinterpret_cast<float*>(a.out)[it] = 0.0f;
      else
        reinterpret_cast<uint16_t*>(a.out)[it] = 0;
    }
    return;
  }

  for (int item = blockIdx.x; item < u * NRB; item += gridDim.x) {
    const int i = item / NRB, rb = item - i * NRB;
    const int e = s.uniq[i];
    const uint32_t mask = s.mask[i];
    const int ntok = __popc(mask);
    const int slot0 = s.off[i];
    const size_t row0 = (size_t)e * H + (size_t)rb * kRows + row_in_item;
    const uint4* W[1] = {reinterpret_cast<const uint4*>(a.wd) + row0 * KU};
    const uint16_t* S[1] = {a.sd + row0 * KG};
    const uint16_t* B[1] = {a.bd + row0 * KG};

    for (int t0 = 0; t0 < ntok; t0 += NT) {
      const int nt = __builtin_amdgcn_readfirstlane(min(NT, ntok - t0));
      __syncthreads();
      if (tid < 32) {
        const int t = (tid < nt) ? nth_set_bit(mask, t0 + tid) : 0;
        toks[tid] = t;
        tokw[tid] = (tid < nt) ? token_expert_weight(a.ids, a.tw, t, k, e) : 0.0f;
      }
      // stage the chunk's hidden vectors (already in pair order) and their sums
      for (int it = tid; it < nt * KU * 8; it += blockDim.x) {
        const int t = it / (KU * 8), rem = it - t * KU * 8;
        const int j = rem >> 3, c = rem & 7;
        const uint4* src = reinterpret_cast<const uint4*>(a.hbuf + ((size_t)(slot0 + t0 + t) * KU + j) * 32);
        act[((size_t)t * 8 + c) * KU + j] = src[c];
      }
      for (int it = tid; it < nt * KU; it += blockDim.x) {
        const int t = it / KU, j = it - t * KU;
        asum[(size_t)t * KU + j] = a.hsum[(size_t)(slot0 + t0 + t) * KU + j];
      }
      __syncthreads();

      float acc[NT][RPG][1];
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < RPG; ++r) acc[t][r][0] = 0.0f;
      rows_dot<LPR, PPL, NT, 1, 8>(W, S, B, KU, KG, act, asum, nt, li, acc);

#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < RPG; ++r) {
          const float y = group_sum<LPR>(acc[t][r][0]);
          if (li == 0 && t < nt)
            a.ys[(size_t)(slot0 + t0 + t) * H + (size_t)rb * kRows + row_in_item + r] = tokw[t] * y;
        }
    }

    // The last of the u work items of this row block adds the experts' parts.
    __threadfence();
    __syncthreads();
    if (tid == 0) *last = (atomicAdd(&a.cnt[rb], 1u) == (uint32_t)(u - 1));
    __syncthreads();
    if (*last) {
      __threadfence();
      for (int it = tid; it < L * kRows; it += blockDim.x) {
        const int t = it / kRows, r = it - t * kRows;
        const size_t m = (size_t)rb * kRows + r;
        float sum = 0.0f;
        for (int i2 = 0; i2 < u; ++i2) {
          const uint32_t mk = s.mask[i2];
          if ((mk >> t) & 1u) {
            const int slot = s.off[i2] + __popc(mk & ((1u << t) - 1u));
            sum += a.ys[(size_t)slot * H + m];
          }
        }
        if (a.out_f32)
          reinterpret_cast<float*>(a.out)[(size_t)t * H + m] = sum;
        else
          reinterpret_cast<uint16_t*>(a.out)[(size_t)t * H + m] = (uint16_t)f32_to_bf16_rne(sum);
      }
      if (tid == 0) a.cnt[rb] = 0u;
    }
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

// positions per lane, rounded up to an instantiated count
int positions_per_lane(int KU, int lpr) {
  const int ppl = (KU + lpr - 1) / lpr;
  static const int kSet[] = {1, 2, 3, 4, 6, 8};
  for (int v : kSet)
    if (ppl <= v) return v;
  return -1;
}

template <template <int, int, int> class K, int LPR, int PPL>
const void* pick_nt(int nt) {
  switch (nt) {
    case 1: return reinterpret_cast<const void*>(&K<LPR, PPL, 1>::fn);
    case 2: return reinterpret_cast<const void*>(&K<LPR, PPL, 2>::fn);
    case 4: return reinterpret_cast<const void*>(&K<LPR, PPL, 4>::fn);
  }
  return nullptr;
}

template <int LPR, int PPL, int NT>
struct GateUpK {
  static void fn(UnionArgs a, dim3 grid, size_t lds, hipStream_t st) {
    hipLaunchKernelGGL((k_gateup<LPR, PPL, NT>), grid, dim3(Tile<LPR>::NTHR), lds, st, a);
  }
};
template <int LPR, int PPL, int NT>
struct DownK {
  static void fn(UnionArgs a, dim3 grid, size_t lds, hipStream_t st) {
    hipLaunchKernelGGL((k_down<LPR, PPL, NT>), grid, dim3(Tile<LPR>::NTHR), lds, st, a);
  }
};

typedef void (*LaunchFn)(UnionArgs, dim3, size_t, hipStream_t);

template <template <int, int, int> class K>
LaunchFn pick(int lpr, int ppl, int nt) {
  const void* f = nullptr;
#define MOEQ4_CASE(L_, P_) \
  if (lpr == L_ && ppl == P_) f = pick_nt<K, L_, P_>(nt);
  MOEQ4_CASE(64, 1) MOEQ4_CASE(64, 2) MOEQ4_CASE(64, 3) MOEQ4_CASE(64, 4) MOEQ4_CASE(64, 6) MOEQ4_CASE(64, 8)
  MOEQ4_CASE(32, 1) MOEQ4_CASE(16, 1) MOEQ4_CASE(8, 1) MOEQ4_CASE(4, 1) MOEQ4_CASE(2, 1)
#undef MOEQ4_CASE
  return reinterpret_cast<LaunchFn>(const_cast<void*>(f));
}

int threads_for(int lpr) {
  switch (lpr) {
    case 64: return Tile<64>::NTHR;
    case 32: return Tile<32>::NTHR;
    case 16: return Tile<16>::NTHR;
    case 8: return Tile<8>::NTHR;
    case 4: return Tile<4>::NTHR;
    case 2: return Tile<2>::NTHR;
  }
  return 0;
}

size_t align16(size_t v) { return (v + 15) & ~size_t(15); }

// LDS layout shared by both kernels: act | asum | hpair | hval | toks | tokw | flag | union
size_t lds_layout(UnionArgs& a, int nt, int nch, int KU) {
  const int P = a.L * a.k;
  const int EW = (a.E + 31) >> 5;
  size_t off = 0;
  a.lds_act = off;   off = align16(off + (size_t)nt * nch * KU * 16);
  a.lds_asum = off;  off = align16(off + (size_t)nt * KU * 4);
  a.lds_hpair = off; off = align16(off + (size_t)nt * kRows * 4);
  a.lds_hval = off;  off = align16(off + (size_t)nt * kRows * 4);
  a.lds_toks = off;  off = align16(off + 32 * 4);
  a.lds_tokw = off;  off = align16(off + 32 * 4);
  a.lds_flag = off;  off = align16(off + 16);
  a.lds_union = off; off = align16(off + (size_t)4 * (2 * EW + 3 * P + 1 + 2));
  return off;
}

constexpr size_t kMaxLds = 160 * 1024;

int pick_nt_for(int L, int nch, int KU, const UnionArgs& a) {
  int nt = L >= 4 ? 4 : (L >= 2 ? 2 : 1);
  while (nt > 1) {
    UnionArgs t = a;
    if (lds_layout(t, nt, nch, KU) <= 64 * 1024) break;
    nt >>= 1;
  }
  return nt;
}

}  // namespace

size_t union_lds_bytes_max(int L, int k, int E, int H, int I) {
  UnionArgs a{};
  a.L = L; a.k = k; a.E = E; a.H = H; a.I = I;
  const size_t g = lds_layout(a, pick_nt_for(L, 4, H / 32, a), 4, H / 32);
  const size_t d = lds_layout(a, pick_nt_for(L, 8, I / 32, a), 8, I / 32);
  return g > d ? g : d;
}

bool union_shape_supported(int L, int k, int E, int H, int I) {
  const int lg = lanes_per_row(H / 32), ld = lanes_per_row(I / 32);
  if (positions_per_lane(H / 32, lg) < 0 || positions_per_lane(I / 32, ld) < 0) return false;
  return union_lds_bytes_max(L, k, E, H, I) <= kMaxLds;
}

int route_union_launch(const int32_t* ids, const float* tw, int L, int k, int E, int32_t* u, int32_t* uniq_ids,
                       uint32_t* tok_mask, float* uniq_w, int32_t* slot_to_uniq, hipStream_t stream) {
  const int P = L * k;
  const int EW = (E + 31) >> 5;
  const int u_max = P < E ? P : E;
  const size_t lds = (size_t)4 * (2 * EW + 3 * P + 1 + 2);
  hipLaunchKernelGGL(k_route_union, dim3(1), dim3(256), lds, stream, ids, tw, L, k, E, u, uniq_ids, tok_mask,
                     uniq_w, slot_to_uniq, u_max);
  return hipGetLastError() == hipSuccess ? MOE_Q4_OK : MOE_Q4_ERR_LAUNCH;
}

int union_forward_launch(const UnionArgs& base, unsigned stages, int num_cu, hipStream_t stream) {
  const int P = base.L * base.k;
  const int u_max = P < base.E ? P : base.E;
  if (stages & MOE_Q4_STAGE_GATEUP) {
    UnionArgs a = base;
    const int KU = a.H / 32;
    const int lpr = lanes_per_row(KU), ppl = positions_per_lane(KU, lpr);
    const int nt = pick_nt_for(a.L, 4, KU, a);
    const size_t lds = lds_layout(a, nt, 4, KU);
    LaunchFn f = pick<GateUpK>(lpr, ppl, nt);
    if (!f || lds > kMaxLds) return MOE_Q4_ERR_UNSUPPORTED;
    const int items = u_max * (a.I / kRows);
    const int per_cu = threads_for(lpr) >= 512 ? 2 : 4;
    int grid = num_cu * per_cu;
    if (grid > items) grid = items;
    if (grid < 1) grid = 1;
    f(a, dim3(grid), lds, stream);
    if (hipGetLastError() != hipSuccess) return MOE_Q4_ERR_LAUNCH;
  }
  if (stages & MOE_Q4_STAGE_DOWN) {
    UnionArgs a = base;
    const int KU = a.I / 32;
    const int lpr = lanes_per_row(KU), ppl = positions_per_lane(KU, lpr);
    const int nt = pick_nt_for(a.L, 8, KU, a);
    const size_t lds = lds_layout(a, nt, 8, KU);
    LaunchFn f = pick<DownK>(lpr, ppl, nt);
    if (!f || lds > kMaxLds) return MOE_Q4_ERR_UNSUPPORTED;
    const int items = u_max * (a.H / kRows);
    const int per_cu = threads_for(lpr) >= 512 ? 2 : 4;
    int grid = num_cu * per_cu;
    if (grid > items) grid = items;
    if (grid < 1) grid = 1;
    f(a, dim3(grid), lds, stream);
    if (hipGetLastError() != hipSuccess) return MOE_Q4_ERR_LAUNCH;
  }
  return MOE_Q4_OK;
}

}  // namespace moeq4
