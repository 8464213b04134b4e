// Matrix-core tiles of the union path for experts that serve many tokens
// (4-bit affine group-64 banks).  Internal header, included by
// moe_q4_union_kernels.h.
//
// When the routes put several tokens on one distinct expert (pooled
// batches: each token takes its experts from a small shared pool, the
// "pooled" rows of the splash PR "perf: Apple7/8 MoE gate and up in one
// decode pass", section "Results"), the per-token dot products of the GEMV
// kernels dominate.  Such an expert's rows are then computed as a small GEMM
// on v_mfma_f32_16x16x32_{bf16,f16}: 16 weight rows x up to 32 tokens, every
// token of the expert in one pass over the weights.
//
// Operands.  A = the tokens (rows of A: the expert's tokens in mask order),
// B = the weight codes (columns of B: 16 consecutive weight rows).  Lane l
// holds A row l % 16 and B column l % 16 over the 8 inputs of lane group
// g = l / 16; the result D[token][row] lands in lane l as tokens
// 4 g .. 4 g + 3 of column (weight row) l % 16.  For each 64-input scale
// group q, lane group g holds the 16 codes 64 q + 16 g .. + 15 of its row
// (see Streaming), and MFMA h = 0, 1 takes the 8 of them at + 8 h: one
// MFMA sums 32 inputs of ONE group, so the group's affine correction
// applies exactly as on the GEMV path:
//     sum_c a_c (s q_c + b) = s * D + (b - M s) * A,  D = sum_c a_c (M + q_c),
// with M + q_c built exactly (M = 128 as bf16 against bf16 activations,
// M = 1024 as fp16 against the fp16 hidden vectors of the down projection)
// and A the sum of the group's 64 activations.  Products are exact and
// accumulate in fp32, as on the GEMV path; only the summation order differs.
// The staged rows of A sit lds_row_units apart in LDS (a pad unit per
// token), so the 16 rows one lane group reads lie in different banks.
//
// Streaming.  Groups go in iterations of 4 (128 bytes of codes per row and
// matrix; scales and biases: one 8-byte piece per array), through a ring of
// three register iterations, two in flight while the third is computed.
// The loads are buffer loads over the tile's 16 rows, so the ring's loads
// past its last step take a zero range and touch no memory (repeating the
// last step instead, issued while it was still in flight, had cost 40-50 %
// extra HBM reads on the pooled batches).
// A lane loads its row's codes as two 16-byte pieces, so one load
// instruction covers 64 contiguous bytes of each of the 16 rows (8-byte
// loads, 32 bytes a row, ran at 1.5 TB/s where these run at 2.3 TB/s, on
// 16 MB of 1 KB rows): piece s of lane group g is words
// 16 s + 8 (g & 1) + 4 (g >> 1) .. + 3 of the iteration's words, that is
// group 2 s + (g & 1)'s words for lane groups g & ~1 (low half) and g | 1
// (high half); each lane keeps its half and trades the other with lane
// l ^ 16 (ds_swizzle), which holds the same group's other half.
// Widths are multiples of 256 (whole iterations) and the scale arrays are
// 8-byte aligned; the host checks both before it launches the kernels that
// hold these tiles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_q4_device.h"
#include "moe_q4_internal.h"

namespace moeq4 {

// Experts with at least this many tokens take the matrix cores, when such
// experts are at least half of the distinct ones (pooled batches).  With
// only a few of them (random routes) the GEMV units stream everything:
// there the tiles would only add a second pipeline fill to the blocks that
// hold them, which then set the kernel's tail.
constexpr int kMfmaMinTokens = 4;
__host__ __device__ constexpr bool mfma_engaged(int many, int u) { return 2 * many >= u && many > 0; }
constexpr int kMfmaRows = 16;  // weight rows of one tile
constexpr int kMfmaGroups = 4;  // scale groups per iteration

typedef __bf16 bf16x8_m_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_m_t __attribute__((ext_vector_type(8)));
typedef float f32x4_m_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_m_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4_m_t mfma16_bf16(uint4 a, uint4 b, f32x4_m_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_m_t, a), __builtin_bit_cast(bf16x8_m_t, b),
                                                 c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_m_t mfma16_f16(uint4 a, uint4 b, f32x4_m_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_m_t, a), __builtin_bit_cast(f16x8_m_t, b), c,
                                                0, 0, 0);
}

__device__ __forceinline__ uint4 unpack_word4(uint32_t w, uint32_t magic) {
  uint32_t q[4];
  unpack_word(w, magic, q);
  return make_uint4(q[0], q[1], q[2], q[3]);
}

typedef unsigned int u32x4_m_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4_m_t bld16m_nt(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_m_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolNt));
}
__device__ __forceinline__ u32x2_m_t bld8m(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2_m_t, bld8(r, off));
}
// Buffer resources over the 16 rows of a tile starting at row rb of a
// matrix of rows of `rowb` code bytes and `G` scale groups; a zero range
// (valid false) turns the loads into no-ops that touch no memory.
struct TileRsrc {
  rsrc_t c, s, b;
};
__device__ __forceinline__ TileRsrc tile_rsrc(const uint32_t* w, const uint16_t* sc, const uint16_t* bi, size_t rb,
                                              int rowb, int G, bool valid) {
  const uint32_t cb = valid ? (uint32_t)(kMfmaRows * rowb) : 0u, sbb = valid ? (uint32_t)(kMfmaRows * G * 2) : 0u;
  return TileRsrc{make_rsrc(reinterpret_cast<const unsigned char*>(w) + rb * rowb, cb),
                  make_rsrc(reinterpret_cast<const unsigned char*>(sc) + rb * G * 2, sbb),
                  make_rsrc(reinterpret_cast<const unsigned char*>(bi) + rb * G * 2, sbb)};
}
// word offset of piece s of lane group g inside an iteration (16 words a
// piece pair)
__device__ __forceinline__ int piece_word(int s, int g) { return 16 * s + 8 * (g & 1) + 4 * (g >> 1); }
// value of lane l ^ 16 (swizzle bit mode: and 0x1F, or 0, xor 0x10)
__device__ __forceinline__ uint32_t swap16(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);
}
// The lane's code pairs of groups 2 s and 2 s + 1 of an iteration (pair c:
// words 8 c + 2 g, + 1 of its row) from its piece s.
__device__ __forceinline__ void piece_pair(const u32x4_m_t& v, int g, u32x2_m_t& p0, u32x2_m_t& p1) {
  const bool odd = g & 1;
  u32x2_m_t own, give, got;
  own.x = odd ? v.z : v.x;
  own.y = odd ? v.w : v.y;
  give.x = odd ? v.x : v.z;
  give.y = odd ? v.y : v.w;
  got.x = swap16(give.x);
  got.y = swap16(give.y);
  p0 = odd ? got : own;
  p1 = odd ? own : got;
}
template <int NP>
__device__ __forceinline__ void piece_pairs(const u32x4_m_t (&v)[NP], int g, u32x2_m_t (&pr)[2 * NP]) {
#pragma unroll
  for (int s = 0; s < NP; ++s) piece_pair(v[s], g, pr[2 * s], pr[2 * s + 1]);
}

// bf16 number i (0..3) of four packed in an 8-byte piece
__device__ __forceinline__ float bf16_of4(u32x2_m_t v, int i) {
  const uint32_t w = (i & 2) ? v.y : v.x;
  return (i & 1) ? bf16_hi_to_f32(w) : bf16_lo_to_f32(w);
}

// The (r)-th token of the expert (mask order); rows past its n tokens repeat
// its first token (their results are dropped).
__device__ __forceinline__ int tile_token(uint32_t mask, int n, int r) { return nth_set_bit(mask, r < n ? r : 0); }

// One iteration (4 groups) of a gate/up tile held by a lane.
struct GuMIt {
  u32x4_m_t cg[2], cu[2];  // codes: the lane's two pieces of its row
  u32x2_m_t sg, bg, su, bu;  // scales and biases of the 4 groups
};

// Gate and up of this block's matrix-core tiles.  The nm distinct experts
// listed in mlist have I / 16 tiles each (16 hidden rows, every token of
// the expert, at most 32); tile t belongs to block t % nblk.  The W waves of
// the block split each tile's inputs: wave w takes iterations w, w + W, ...
// (256 inputs each), and the waves' partial sums meet in LDS (red,
// [W][8][64] fp32) where they are added in wave order, one 16-token block
// at a time, before h = silu(gate) * up goes to hbuf[(slot0 + r) * I + row]
// for the token of rank r.  Each wave streams its share of the block's
// tiles through one ring of three register iterations, so the next tile's
// loads are in flight across a reduction's barriers.  Every wave of the
// block runs the same steps (the barriers are block-uniform).
// act / asum: the staged activations (pair order per 8 inputs, rows
// lds_row_units(H) apart) and their 32-input sums ([L][H / 32]).
template <int W>
__device__ inline void gu_mfma_phase(const UnionArgs& a, const UnionLds& s, const int* mlist, int nm, const uint4* act,
                                     const float* asum, float* red, int b, int nblk) {
  const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int H = a.H, I = a.I, G = H >> 6, nit = G / kMfmaGroups, KU = H >> 5, TS = lds_row_units(H);
  const int tpe = I / kMfmaRows, ntm = nm * tpe;
  const int ntb = ntm > b ? (ntm - 1 - b) / nblk + 1 : 0;  // tiles of this block
  const int spw = (nit + W - 1) / W;                        // steps of a wave per tile
  const int Z = ntb * spw;
  if (Z == 0) return;  // uniform over the block
  // tile j of the block: distinct expert index i and first hidden row
  auto tile = [&](int j, int& i, int& row0) {
    const int t = b + j * nblk, x = t / tpe;
    i = __builtin_amdgcn_readfirstlane(mlist[x]);
    row0 = (t - x * tpe) * kMfmaRows;
  };
  // step z: iteration wave + W (z % spw) of tile z / spw; steps past the
  // end and iterations past the row are zero-range no-ops, so every load
  // is unconditional and none re-reads memory
  auto load = [&](int z, GuMIt& f) {
    const int zz = min(z, Z - 1), j = zz / spw;
    const int itr = wave + W * (zz - j * spw);
    const bool valid = z < Z && itr < nit;
    const int it = min(itr, nit - 1);
    int i, row0;
    tile(j, i, row0);
    const size_t rb = (size_t)__builtin_amdgcn_readfirstlane(s.uniq[i]) * I + row0;
    const TileRsrc tg = tile_rsrc(a.wg, a.sg, a.bg, rb, H / 2, G, valid);
    const TileRsrc tu = tile_rsrc(a.wu, a.su, a.bu, rb, H / 2, G, valid);
    const uint32_t coff = (uint32_t)(m * (H / 2) + 128 * it);
    const uint32_t soff = (uint32_t)((m * G + kMfmaGroups * it) * 2);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      f.cg[c] = bld16m_nt(tg.c, coff + 4 * piece_word(c, g));
      f.cu[c] = bld16m_nt(tu.c, coff + 4 * piece_word(c, g));
    }
    f.sg = bld8m(tg.s, soff);
    f.bg = bld8m(tg.b, soff);
    f.su = bld8m(tu.s, soff);
    f.bu = bld8m(tu.b, soff);
  };
  // the current tile
  int ta[2], tc[2][4], n = 0, slot0 = 0, crow0 = 0;
  float og[2][4], ou[2][4];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int v = 0; v < 4; ++v) og[tb][v] = ou[tb][v] = 0.0f;
  auto finish = [&]() {
    const int nb = n > 16 ? 2 : 1;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      if (tb < nb) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          red[(wave * 8 + v) * 64 + lane] = og[tb][v];
          red[(wave * 8 + 4 + v) * 64 + lane] = ou[tb][v];
        }
        __syncthreads();
        if (threadIdx.x < 256) {
          const int l = threadIdx.x & 63, v = threadIdx.x >> 6;
          float gs = 0.0f, us = 0.0f;
#pragma unroll
          for (int w = 0; w < W; ++w) {
            gs += red[(w * 8 + v) * 64 + l];
            us += red[(w * 8 + 4 + v) * 64 + l];
          }
          const int r = 16 * tb + 4 * (l >> 4) + v;
          if (r < n)
            a.hbuf[(size_t)(slot0 + r) * I + crow0 + (l & 15)] = gs * __builtin_amdgcn_rcpf(1.0f + __expf(-gs)) * us;
        }
        __syncthreads();
      }
    }
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int v = 0; v < 4; ++v) og[tb][v] = ou[tb][v] = 0.0f;
  };
  auto compute = [&](int z, const GuMIt& f) {
    const int j = z / spw, sidx = z - j * spw;
    if (sidx == 0) {
      int i;
      tile(j, i, crow0);
      const uint32_t mask = (uint32_t)__builtin_amdgcn_readfirstlane((int)s.mask[i]);
      n = __popc(mask);
      slot0 = __builtin_amdgcn_readfirstlane(s.off[i]);
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        ta[tb] = tile_token(mask, n, 16 * tb + m);
#pragma unroll
        for (int v = 0; v < 4; ++v) tc[tb][v] = tile_token(mask, n, 16 * tb + 4 * g + v);
      }
    }
    const int it = wave + W * sidx;
    if (it < nit) {
      const int nb = n > 16 ? 2 : 1;
      u32x2_m_t pg[kMfmaGroups], pu[kMfmaGroups];
      piece_pairs<2>(f.cg, g, pg);
      piece_pairs<2>(f.cu, g, pu);
#pragma unroll
      for (int c = 0; c < kMfmaGroups; ++c) {
        const int q = kMfmaGroups * it + c;
        const float s_g = bf16_of4(f.sg, c), s_u = bf16_of4(f.su, c);
        const float c_g = bf16_of4(f.bg, c) - 128.0f * s_g, c_u = bf16_of4(f.bu, c) - 128.0f * s_u;
        const uint4 bg0 = unpack_word4(pg[c].x, kMagicBytes), bg1 = unpack_word4(pg[c].y, kMagicBytes);
        const uint4 bu0 = unpack_word4(pu[c].x, kMagicBytes), bu1 = unpack_word4(pu[c].y, kMagicBytes);
        // activations 64 q + 16 g + 8 h .. + 7: position 2 q + g / 2, 8-block (2 g + h) % 4
        const int pos = 2 * q + (g >> 1);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          if (tb < nb) {
            const uint4* ar = act + (size_t)ta[tb] * TS + pos;
            const uint4 a0 = ar[((2 * g) & 3) * KU], a1 = ar[((2 * g + 1) & 3) * KU];
            f32x4_m_t dg = {0.0f, 0.0f, 0.0f, 0.0f}, du = {0.0f, 0.0f, 0.0f, 0.0f};
            dg = mfma16_bf16(a0, bg0, dg);
            du = mfma16_bf16(a0, bu0, du);
            dg = mfma16_bf16(a1, bg1, dg);
            du = mfma16_bf16(a1, bu1, du);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float2 sx = *reinterpret_cast<const float2*>(asum + (size_t)tc[tb][v] * KU + 2 * q);
              const float xs = sx.x + sx.y;
              og[tb][v] += s_g * dg[v] + c_g * xs;
              ou[tb][v] += s_u * du[v] + c_u * xs;
            }
          }
        }
      }
    }
    if (sidx == spw - 1) finish();
  };
  GuMIt f0, f1, f2;
  load(0, f0);
  load(1, f1);
#pragma unroll 1
  for (int z = 0;; z += 3) {
    load(z + 2, f2);
    compute(z, f0);
    if (z + 1 >= Z) break;
    load(z + 3, f0);
    compute(z + 1, f1);
    if (z + 2 >= Z) break;
    load(z + 4, f1);
    compute(z + 2, f2);
    if (z + 3 >= Z) break;
  }
}

// One iteration (4 groups) of a down tile held by a lane.
struct DnMIt {
  u32x4_m_t c[2];  // codes: the lane's two pieces of its row
  u32x2_m_t s, b;  // scales and biases of the 4 groups
};

// A down tile: 16 output rows (r0 ..) of distinct expert e for its tokens
// staged in LDS slots ls0 .. ls0 + n - 1 (1 <= n <= 32).
struct DnTile {
  int e, r0, ls0, n;
};

// The down tiles of one wave: tasks j0, j0 + stride, ... below jend, of
// which tile(j, t) marks the tiles (and fills t).  All of them stream
// through one ring of three register iterations, so the next tile's loads
// are in flight while a tile finishes.  The slots hold the hidden vectors
// as fp16 (pair order per 8 inputs, rows lds_row_units(I) apart), their
// 32-input sums hss ([slot][I / 32]), router weights stw, ys rows sdst and
// scaling exponents sexp; each token's 16 outputs, times its router weight
// and shifted back by its exponent, go to its ys row.
template <typename TileFn>
__device__ inline void dn_mfma_run(const UnionArgs& a, TileFn&& tile, int j0, int stride, int jend, const uint4* hvs,
                                   const float* hss, const float* stw, const int* sdst, const int* sexp) {
  const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
  const int H = a.H, I = a.I, G = I >> 6, nit = G / kMfmaGroups, KU = I >> 5, TS = lds_row_units(I);
  // a position in the wave's step sequence: task j, iteration it of its tile
  struct Cur {
    int j, it;
    bool done;
    DnTile t;
  };
  auto first = [&](int j, DnTile& t) {
    for (; j < jend; j += stride)
      if (tile(j, t)) break;
    return j;
  };
  Cur lc;
  lc.j = first(j0, lc.t);
  lc.it = 0;
  lc.done = false;
  if (lc.j >= jend) return;
  Cur cc = lc;
  // one step on; past the last tile a cursor stays on that tile's last
  // iteration and reports false (its loads are then zero-range no-ops)
  auto step = [&](Cur& c) {
    if (c.done) return false;
    if (++c.it < nit) return true;
    DnTile t;
    const int j = first(c.j + stride, t);
    if (j >= jend) {
      c.it = nit - 1;
      c.done = true;
      return false;
    }
    c.j = j;
    c.it = 0;
    c.t = t;
    return true;
  };
  auto load = [&](const Cur& c, DnMIt& f) {
    const size_t rb = (size_t)c.t.e * H + c.t.r0;
    const TileRsrc td = tile_rsrc(a.wd, a.sd, a.bd, rb, I / 2, G, !c.done);
    const uint32_t coff = (uint32_t)(m * (I / 2) + 128 * c.it);
    const uint32_t soff = (uint32_t)((m * G + kMfmaGroups * c.it) * 2);
#pragma unroll
    for (int k = 0; k < 2; ++k) f.c[k] = bld16m_nt(td.c, coff + 4 * piece_word(k, g));
    f.s = bld8m(td.s, soff);
    f.b = bld8m(td.b, soff);
  };
  int la[2], lt[2][4], nb = 1;
  float o[2][4];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int v = 0; v < 4; ++v) o[tb][v] = 0.0f;
  auto compute = [&](const Cur& c, const DnMIt& f) {
    const int ls0 = c.t.ls0, n = c.t.n;
    if (c.it == 0) {
      nb = n > 16 ? 2 : 1;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        la[tb] = ls0 + min(16 * tb + m, n - 1);
#pragma unroll
        for (int v = 0; v < 4; ++v) lt[tb][v] = ls0 + min(16 * tb + 4 * g + v, n - 1);
      }
    }
    u32x2_m_t pd[2];  // one piece's pairs at a time: fewer live registers
#pragma unroll
    for (int k = 0; k < kMfmaGroups; ++k) {
      if ((k & 1) == 0) piece_pair(f.c[k >> 1], g, pd[0], pd[1]);
      const int q = kMfmaGroups * c.it + k;
      const float sc = bf16_of4(f.s, k);
      const float cb = bf16_of4(f.b, k) - 1024.0f * sc;
      const uint4 b0 = unpack_word4(pd[k & 1].x, kMagicBytesF16), b1 = unpack_word4(pd[k & 1].y, kMagicBytesF16);
      const int pos = 2 * q + (g >> 1);
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        if (tb < nb) {
          const uint4* hr = hvs + (size_t)la[tb] * TS + pos;
          const uint4 h0 = hr[((2 * g) & 3) * KU], h1 = hr[((2 * g + 1) & 3) * KU];
          f32x4_m_t d = {0.0f, 0.0f, 0.0f, 0.0f};
          d = mfma16_f16(h0, b0, d);
          d = mfma16_f16(h1, b1, d);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float2 sh = *reinterpret_cast<const float2*>(hss + (size_t)lt[tb][v] * KU + 2 * q);
            o[tb][v] += sc * d[v] + cb * (sh.x + sh.y);
          }
        }
      }
    }
    if (c.it == nit - 1) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = 16 * tb + 4 * g + v;
          if (tb < nb && r < n) {
            const int ls = ls0 + r;
            a.ys[(size_t)sdst[ls] * H + c.t.r0 + m] = __builtin_amdgcn_ldexpf(stw[ls] * o[tb][v], sexp[ls]);
          }
          o[tb][v] = 0.0f;
        }
    }
  };
  DnMIt f0, f1, f2;
  load(lc, f0);
  step(lc);
  load(lc, f1);
  step(lc);
#pragma unroll 1
  for (;;) {
    load(lc, f2);
    step(lc);
    compute(cc, f0);
    if (!step(cc)) break;
    load(lc, f0);
    step(lc);
    compute(cc, f1);
    if (!step(cc)) break;
    load(lc, f1);
    step(lc);
    compute(cc, f2);
    if (!step(cc)) break;
  }
}

}  // namespace moeq4
