// Sorted grouped path of the SwitchGLU-q4 MoE layer for gfx950 (MI355X), used
// when the token count is too large for the union path (prefill).
//
// Sources (web pages): sorting the (token, expert) pairs by expert and running
// a grouped matmul over expert-contiguous rows is the sorted gather path of the
// page "MoE GatherQMM small-M verify cost" (Facts: the gather_qmm_rhs
// dispatch and its sorted_indices condition); cutting row tiles at expert
// boundaries, ceil(n_e / BM) tiles per expert, is the tile scheduler of PR
// 4567 / PR 4572 described on the same page; the SwitchGLU order (up, gate,
// silu(gate) * up, down) follows the moe_bench script of the mlx issue
// "gather_qmm at M=1 streams 4-bit expert weights at ~half the bandwidth of
// M=4".
//
// One forward = six launches on one stream:
//   k_sort_scan      one workgroup: per-expert counts, exclusive scan ->
//                    offsets[E+1], the tile list, and an unordered scatter of
//                    the pairs into their expert's segment.
//   k_sort_rank      one thread per pair: its rank by pair index inside its
//                    expert's segment, which makes the order stable (sorted by
//                    (expert, pair)) -> perm and inv.
//   k_token_gsum     per token and 64-input group, the fp32 sum of x; per
//                    token the exponent e_t of its largest |x| (h is stored
//                    times 2^-e_t and the combine undoes it exactly).
//   k_sorted_gateup  per (tile, 128 hidden columns): the tile's gathered x rows
//                    staged in LDS per 64-input group; gate and up codes go
//                    straight from HBM into registers and become exact bf16
//                    (128 + q) MFMA operands; one v_mfma_f32_32x32x16_bf16
//                    chain per group and 32x32 block, then the group's affine
//                    correction in fp32:
//                        sum_c x_c (s q_c + b) = s * D + (b - 128 s) * A,
//                        D = sum_c x_c (128 + q_c),  A = sum_c x_c;
//                    h = silu(gate) * up is written as a bf16 hi + lo pair
//                    (h - hi rounded again), plus per-32-column sums of hi + lo.
//   k_sorted_down    per (tile, 256 output columns): A = h hi and h lo (two
//                    MFMA passes on the same codes), same affine correction
//                    with the staged sums of hi + lo -> one fp32 output row per
//                    pair.
//   k_sorted_combine out[t] = sum over t's slots j (ascending) of w[t, j] *
//                    y[inv(t, j)]: deterministic, no floating-point atomics.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "moe_q4.h"
#include "moe_q4_device.h"
#include "moe_q4_internal.h"

namespace moeq4 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kSortThreads = 1024;
constexpr int kMmThreads = 256;       // 4 waves per GEMM workgroup
constexpr int kRowTile = 32;          // rows of one MFMA block
constexpr int kGuCols = 128;          // hidden columns of one gate/up workgroup (32 per wave)
constexpr int kDnCols = 256;          // output columns of one down workgroup (64 per wave)
constexpr int kRowBytes = 144;        // LDS bytes per staged row: 8 x 16 B of one group + 16 B pad

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ uint4 unpack_codes(uint32_t w) {
  uint32_t q[4];
  unpack_word(w, kMagicBytes, q);
  return make_uint4(q[0], q[1], q[2], q[3]);
}

__device__ __forceinline__ f32x16_t mfma_bf16(uint4 a, uint4 b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// sort
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kSortThreads) void k_sort_scan(SortedArgs a) {
  extern __shared__ __align__(16) int32_t sl[];
  const int P = a.T * a.k, E = a.E, tid = threadIdx.x;
  int32_t* cnt = sl;                    // [E+1] counts, then scatter cursors
  int32_t* part = sl + E + 1;           // [1024] per-thread pair sums
  int32_t* tpart = part + kSortThreads; // [1024] per-thread tile sums
  __shared__ int bad;
  for (int e = tid; e <= E; e += kSortThreads) cnt[e] = 0;
  if (tid == 0) bad = 0;
  __syncthreads();
  for (int p = tid; p < P; p += kSortThreads) {
    const int e = a.ids[p];
    const bool ok = e >= 0 && e < E;
    if (!ok) bad = 1;
    atomicAdd(&cnt[ok ? e : E], 1);
  }
  __syncthreads();
  // each thread scans a contiguous run of keys (key E collects invalid ids)
  const int n = E + 1;
  const int per = (n + kSortThreads - 1) / kSortThreads;
  const int c0 = min(n, tid * per), c1 = min(n, c0 + per);
  int s = 0, ts = 0;
  for (int e = c0; e < c1; ++e) {
    s += cnt[e];
    if (e < E) ts += (cnt[e] + a.bm - 1) / a.bm;
  }
  part[tid] = s;
  tpart[tid] = ts;
  __syncthreads();
  for (int d = 1; d < kSortThreads; d <<= 1) {
    int v = 0, tv = 0;
    if (tid >= d) {
      v = part[tid - d];
      tv = tpart[tid - d];
    }
    __syncthreads();
    if (tid >= d) {
      part[tid] += v;
      tpart[tid] += tv;
    }
    __syncthreads();
  }
  int run = tid ? part[tid - 1] : 0;
  int trun = tid ? tpart[tid - 1] : 0;
  for (int e = c0; e < c1; ++e) {
    const int c = cnt[e];
    a.offsets[e] = run;  // offsets[E] = number of valid pairs
    if (e < E)
      for (int r = 0; r < c; r += a.bm) a.tiles[trun++] = make_int4(e, run + r, min(a.bm, c - r), 0);
    cnt[e] = run;
    run += c;
  }
  __syncthreads();
  if (tid == 0) {
    a.hdr[0] = bad ? MOE_Q4_DEV_BAD_ID : 0u;
    a.hdr[1] = MOE_Q4_PATH_SORTED;
    a.hdr[2] = (uint32_t)cnt[E];
    a.hdr[3] = (uint32_t)tpart[kSortThreads - 1];
  }
  __syncthreads();  // cnt[E] read above before the scatter moves the cursors
  for (int p = tid; p < P; p += kSortThreads) {
    const int e = a.ids[p];
    const int key = (e >= 0 && e < E) ? e : E;
    a.rank_tmp[atomicAdd(&cnt[key], 1)] = p;
  }
}

__global__ __launch_bounds__(256) void k_sort_rank(SortedArgs a) {
  const int P = a.T * a.k;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= P) return;
  const int p = a.rank_tmp[i];
  const int e = a.ids[p];
  const bool ok = e >= 0 && e < a.E;
  const int lo = ok ? a.offsets[e] : a.offsets[a.E];
  const int hi = ok ? a.offsets[e + 1] : P;
  int r = 0;
  for (int j = lo; j < hi; ++j) r += a.rank_tmp[j] < p;
  a.perm[lo + r] = p;
  a.inv[p] = lo + r;
}

// Per token: the fp32 sum of x over each 64-input group (affine banks only),
// and the exponent e_t of the token's largest |x|.  The gate/up kernels
// store h * 2^-e_t and the combine multiplies the token's output by 2^e_t
// (both exact), so the bf16 hi + lo planes of h stay in the normal range for
// tokens with tiny activations: h scales like x^2, and below about 2^-117
// the lo plane would be subnormal, which the MFMAs flush to zero.
__global__ __launch_bounds__(256) void k_token_gsum(SortedArgs a) {
  const int t = blockIdx.x;
  const int G = a.H / 64;
  uint32_t mb = 0;  // largest |x| as bf16 magnitude bits (they order like the values)
  for (int g = threadIdx.x; g < G; g += 256) {
    const uint4* src = reinterpret_cast<const uint4*>(a.x + (size_t)t * a.H + 64 * g);
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint4 v = src[c];
      acc = sum8_bf16(v, acc);
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) mb = max(mb, max(w4[q] & 0x7FFFu, (w4[q] >> 16) & 0x7FFFu));
    }
    if (a.fmt == kFmtAffine) a.asum[(size_t)t * G + g] = acc;
  }
  __shared__ uint32_t wmax[4];
  float m = __uint_as_float(mb << 16);
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = __float_as_uint(m);
  __syncthreads();
  if (threadIdx.x == 0) {
    const float mx = fmaxf(fmaxf(__uint_as_float(wmax[0]), __uint_as_float(wmax[1])),
                           fmaxf(__uint_as_float(wmax[2]), __uint_as_float(wmax[3])));
    a.texp[t] = mx > 0.0f ? __builtin_amdgcn_frexp_expf(mx) : 0;
  }
}

// ---------------------------------------------------------------------------
// block index -> (tile, column block): the column blocks of one tile run on
// one XCD back to back (block b lands on XCD b % 8), so the tile's staged rows
// are read from that XCD's L2 after the first block.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void tile_of_block(int ncb, int& tile, int& cb) {
  const int b = blockIdx.x;
  const int x = b & 7, j = b >> 3;
  tile = x + 8 * (j / ncb);
  cb = j % ncb;
}

// Row of the 32x32 MFMA result held in element i of lane half hh.
__device__ __forceinline__ int c_row(int i, int hh) { return 8 * (i >> 2) + 4 * hh + (i & 3); }

// ---------------------------------------------------------------------------
// gate + up
// ---------------------------------------------------------------------------

struct GuFragS {
  uint4 g, u;       // this lane's 4 code words of gate and up (one half of the group)
  uint32_t sb[4];   // bf16 sg, bg, su, bu of this lane's column
};

template <int MT>
__global__ __launch_bounds__(kMmThreads, 2) void k_sorted_gateup(SortedArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int H = a.H, I = a.I, G = H / 64;
  const int ncb = (I + kGuCols - 1) / kGuCols;
  int tile, cb;
  tile_of_block(ncb, tile, cb);
  if (tile >= (int)a.hdr[3]) return;
  const int4 td = a.tiles[tile];
  const int e = td.x, r0 = td.y, nrows = td.z;
  const int nrt = (nrows + kRowTile - 1) / kRowTile;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, hh = lane >> 5, lc = lane & 31;
  const int col0 = cb * kGuCols + 32 * wid;
  const bool wave_on = col0 < I;
  const int col = wave_on ? col0 + lc : 0;

  constexpr int kRows = MT * kRowTile;
  unsigned char* abuf = smem;                                      // [2][kRows][kRowBytes]
  float* sbuf = reinterpret_cast<float*>(smem + 2 * kRows * kRowBytes);  // [2][kRows]
  int32_t* tok = reinterpret_cast<int32_t*>(sbuf + 2 * kRows);    // [kRows]

  for (int r = tid; r < kRows; r += kMmThreads) tok[r] = a.perm[r0 + min(r, nrows - 1)] / a.k;
  __syncthreads();

  // staging of one group of the tile's x rows (codes order) and their sums
  constexpr int kPer = kRows * 8 / kMmThreads;  // uint4 per thread
  uint4 st[kPer];
  float sst = 0.0f;
  // every thread loads unconditionally (rows past the tile repeat its last
  // row: same addresses, no extra HBM traffic), so the waits stay exact
  auto stage_load = [&](int g) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = tid + kMmThreads * i, r = idx >> 3, w = idx & 7;
      st[i] = *reinterpret_cast<const uint4*>(a.x + (size_t)tok[r] * H + 64 * g + 8 * w);
    }
    sst = a.asum[(size_t)tok[min(tid, kRows - 1)] * G + g];
  };
  auto stage_store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = tid + kMmThreads * i, r = idx >> 3, w = idx & 7;
      *reinterpret_cast<uint4*>(abuf + (size_t)(buf * kRows + r) * kRowBytes + 16 * w) = pair_activations(st[i]);
    }
    if (tid < kRows) sbuf[buf * kRows + tid] = sst;
  };

  const size_t rowg = ((size_t)e * I + col) * (size_t)(H / 8);
  const size_t rows = ((size_t)e * I + col) * (size_t)G;
  auto frag_load = [&](int g) {
    GuFragS f;
    f.g = *reinterpret_cast<const uint4*>(a.wg + rowg + 8 * g + 4 * hh);
    f.u = *reinterpret_cast<const uint4*>(a.wu + rowg + 8 * g + 4 * hh);
    f.sb[0] = a.sg[rows + g];
    f.sb[1] = a.bg[rows + g];
    f.sb[2] = a.su[rows + g];
    f.sb[3] = a.bu[rows + g];
    return f;
  };

  f32x16_t og[MT], ou[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) og[m][i] = ou[m][i] = 0.0f;

  GuFragS f0 = frag_load(0), f1 = frag_load(min(1, G - 1));
  stage_load(0);
  stage_store(0);
  __syncthreads();

  for (int g = 0; g < G; ++g) {
    const int buf = g & 1;
    const GuFragS f2 = frag_load(min(g + 2, G - 1));
    stage_load(min(g + 1, G - 1));
    if (wave_on) {
      const uint32_t wg4[4] = {f0.g.x, f0.g.y, f0.g.z, f0.g.w};
      const uint32_t wu4[4] = {f0.u.x, f0.u.y, f0.u.z, f0.u.w};
      uint4 bg_[4], bu_[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bg_[s] = unpack_codes(wg4[s]);
        bu_[s] = unpack_codes(wu4[s]);
      }
      const float s_g = bf16_to_f32((uint16_t)f0.sb[0]), b_g = bf16_to_f32((uint16_t)f0.sb[1]) - 128.0f * s_g;
      const float s_u = bf16_to_f32((uint16_t)f0.sb[2]), b_u = bf16_to_f32((uint16_t)f0.sb[3]) - 128.0f * s_u;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < nrt) {
          const unsigned char* arow = abuf + (size_t)(buf * kRows + m * kRowTile + lc) * kRowBytes + 64 * hh;
          uint4 av[4];
#pragma unroll
          for (int s = 0; s < 4; ++s) av[s] = *reinterpret_cast<const uint4*>(arow + 16 * s);
          f32x16_t pg = {}, pu = {};
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            pg = mfma_bf16(av[s], bg_[s], pg);
            pu = mfma_bf16(av[s], bu_[s], pu);
          }
          const float* srow = sbuf + buf * kRows + m * kRowTile + 4 * hh;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 sa = *reinterpret_cast<const float4*>(srow + 8 * q);
            const float sv[4] = {sa.x, sa.y, sa.z, sa.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int i = 4 * q + r;
              og[m][i] = fmaf(b_g, sv[r], fmaf(s_g, pg[i], og[m][i]));
              ou[m][i] = fmaf(b_u, sv[r], fmaf(s_u, pu[i], ou[m][i]));
            }
          }
        }
      }
    }
    stage_store(buf ^ 1);
    __syncthreads();
    f0 = f1;
    f1 = f2;
  }

  if (!wave_on) return;
  // h = silu(gate) * up; stored as bf16 hi + lo in code order within each 8 columns
  const int scol = (col & ~7) | ((col & 7) >> 1) | ((col & 1) << 2);
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m < nrt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = m * kRowTile + c_row(i, hh);
        const float gv = og[m][i];
        const float hv = __builtin_amdgcn_ldexpf(gv / (1.0f + __expf(-gv)) * ou[m][i], -a.texp[tok[r]]);
        const uint32_t hi = f32_to_bf16_rne(hv);
        const float hif = __uint_as_float(hi << 16);
        const uint32_t lo = f32_to_bf16_rne(hv - hif);
        const float v = group_sum<32>(hif + __uint_as_float(lo << 16));
        if (r < nrows) {
          const size_t o = (size_t)(r0 + r) * I;
          a.hhi[o + scol] = (uint16_t)hi;
          a.hlo[o + scol] = (uint16_t)lo;
          if (lc == 0) a.hsum2[(size_t)(r0 + r) * (I / 32) + col0 / 32] = v;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// down
// ---------------------------------------------------------------------------

struct DnFragS {
  uint4 w0, w1;     // this lane's 4 code words for each of its two 32-column blocks
  uint32_t s0, b0, s1, b1;  // bf16 sd, bd of both columns
};

template <int MT>
__global__ __launch_bounds__(kMmThreads, 2) void k_sorted_down(SortedArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int H = a.H, I = a.I, G = I / 64;
  const int ncb = (H + kDnCols - 1) / kDnCols;
  int tile, cb;
  tile_of_block(ncb, tile, cb);
  if (tile >= (int)a.hdr[3]) return;
  const int4 td = a.tiles[tile];
  const int e = td.x, r0 = td.y, nrows = td.z;
  const int nrt = (nrows + kRowTile - 1) / kRowTile;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, hh = lane >> 5, lc = lane & 31;
  const int colw = cb * kDnCols + 64 * wid;  // first column of this wave
  bool on[2];
  int col[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    on[c] = colw + 32 * c < H;
    col[c] = on[c] ? colw + 32 * c + lc : 0;
  }

  constexpr int kRows = MT * kRowTile;
  unsigned char* abuf = smem;  // [2 buffers][2 planes][kRows][kRowBytes]
  float* sbuf = reinterpret_cast<float*>(smem + 4 * kRows * kRowBytes);  // [2][kRows]

  constexpr int kPer = kRows * 8 / kMmThreads;  // 16-byte pieces per thread and plane
  u32x4_t sth[kPer], stl[kPer];
  float sst = 0.0f;
  // unconditional loads (rows past the tile repeat its last row), exact waits
  auto stage_load = [&](int g) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = tid + kMmThreads * i, r = min(idx >> 3, nrows - 1), w = idx & 7;
      const size_t o = (size_t)(r0 + r) * I + 64 * g + 8 * w;
      sth[i] = *reinterpret_cast<const u32x4_t*>(a.hhi + o);
      stl[i] = *reinterpret_cast<const u32x4_t*>(a.hlo + o);
    }
    const float* hs = a.hsum2 + (size_t)(r0 + min(tid, nrows - 1)) * (I / 32) + 2 * g;
    sst = hs[0] + hs[1];
  };
  auto stage_store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = tid + kMmThreads * i, r = idx >> 3, w = idx & 7;
      *reinterpret_cast<u32x4_t*>(abuf + (size_t)((buf * 2 + 0) * kRows + r) * kRowBytes + 16 * w) = sth[i];
      *reinterpret_cast<u32x4_t*>(abuf + (size_t)((buf * 2 + 1) * kRows + r) * kRowBytes + 16 * w) = stl[i];
    }
    if (tid < kRows) sbuf[buf * kRows + tid] = sst;
  };

  size_t rw[2], rs[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    rw[c] = ((size_t)e * H + col[c]) * (size_t)(I / 8);
    rs[c] = ((size_t)e * H + col[c]) * (size_t)G;
  }
  auto frag_load = [&](int g) {
    DnFragS f;
    f.w0 = *reinterpret_cast<const uint4*>(a.wd + rw[0] + 8 * g + 4 * hh);
    f.w1 = *reinterpret_cast<const uint4*>(a.wd + rw[1] + 8 * g + 4 * hh);
    f.s0 = a.sd[rs[0] + g];
    f.b0 = a.bd[rs[0] + g];
    f.s1 = a.sd[rs[1] + g];
    f.b1 = a.bd[rs[1] + g];
    return f;
  };

  f32x16_t acc[MT][2];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][c][i] = 0.0f;

  DnFragS f0 = frag_load(0), f1 = frag_load(min(1, G - 1));
  stage_load(0);
  stage_store(0);
  __syncthreads();

  for (int g = 0; g < G; ++g) {
    const int buf = g & 1;
    const DnFragS f2 = frag_load(min(g + 2, G - 1));
    stage_load(min(g + 1, G - 1));
    uint4 bw[2][4];
    float sc[2], bc[2];
    {
      const uint32_t w8[8] = {f0.w0.x, f0.w0.y, f0.w0.z, f0.w0.w, f0.w1.x, f0.w1.y, f0.w1.z, f0.w1.w};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bw[0][s] = unpack_codes(w8[s]);
        bw[1][s] = unpack_codes(w8[4 + s]);
      }
      sc[0] = bf16_to_f32((uint16_t)f0.s0);
      bc[0] = bf16_to_f32((uint16_t)f0.b0) - 128.0f * sc[0];
      sc[1] = bf16_to_f32((uint16_t)f0.s1);
      bc[1] = bf16_to_f32((uint16_t)f0.b1) - 128.0f * sc[1];
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m < nrt) {
        uint4 ahi[4], alo[4];
        const unsigned char* ph = abuf + (size_t)((buf * 2 + 0) * kRows + m * kRowTile + lc) * kRowBytes + 64 * hh;
        const unsigned char* pl = abuf + (size_t)((buf * 2 + 1) * kRows + m * kRowTile + lc) * kRowBytes + 64 * hh;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          ahi[s] = *reinterpret_cast<const uint4*>(ph + 16 * s);
          alo[s] = *reinterpret_cast<const uint4*>(pl + 16 * s);
        }
        const float* srow = sbuf + buf * kRows + m * kRowTile + 4 * hh;
        float sv[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 sa = *reinterpret_cast<const float4*>(srow + 8 * q);
          sv[4 * q] = sa.x; sv[4 * q + 1] = sa.y; sv[4 * q + 2] = sa.z; sv[4 * q + 3] = sa.w;
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          if (on[c]) {
            f32x16_t p = {};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              p = mfma_bf16(ahi[s], bw[c][s], p);
              p = mfma_bf16(alo[s], bw[c][s], p);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[m][c][i] = fmaf(bc[c], sv[i], fmaf(sc[c], p[i], acc[m][c][i]));
          }
        }
      }
    }
    stage_store(buf ^ 1);
    __syncthreads();
    f0 = f1;
    f1 = f2;
  }

#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m < nrt) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        if (on[c]) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int r = m * kRowTile + c_row(i, hh);
            if (r < nrows) a.ys[(size_t)(r0 + r) * H + col[c]] = acc[m][c][i];
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// streaming variants for the common shapes (H, I multiples of 1024)
//
// The kernels above give each lane 16 bytes of one weight row per 64-input
// group and 2 bytes of its scale row, so every 128-byte line is touched many
// times, far apart in time, by 128 columns in flight per workgroup -- more
// lines than L2 holds, and each touch refetches the line.  These variants
// consume whole lines at once: an iteration covers 4 groups (the two halves
// of a 32-lane column group read a row's full 128-byte code line), scales and
// biases arrive 16 groups (32 bytes) per load, and gate and up run on
// separate waves, which halves each wave's registers.  x (or h) staging loads
// are issued before the weight prefetch of the same iteration, so the wait
// for the staged rows never waits for weights still in flight.
// ---------------------------------------------------------------------------

constexpr int kV2Threads = 512;              // 8 waves
constexpr int kV2GuCols = 128;               // gate/up: waves 0-3 gate, 4-7 up, 32 columns each
constexpr int kV2DnCols = 256;               // down: 8 waves x 32 columns
constexpr int kV2Row = 4 * 128 + 16;         // LDS bytes per staged row: 4 groups + pad

struct Chunk16 {
  uint4 s0, s1, b0, b1;  // 16 consecutive bf16 scales and biases of one row
};

// The affine correction's second half on the matrix cores.  Per 64-input
// group g the layer needs out += s_g * P_g + (b_g - 128 s_g) * A_g (P_g the
// group's MFMA chain over the 128 + q operands, A_g the rows' input sums).
// The s_g * P_g half stays a per-group fp32 FMA; the other half is, over
// the 16 groups of a chunk, a product with K = 16 groups: A (rows x groups)
// times b and times -128 s (groups x columns).  b and -128 s are exact bf16
// operands; A is fp32, so it enters as three bf16 planes whose sum is A to
// within 2^-27 of it.  This takes the per-group row-sum reads (as many LDS
// bytes as the activation operands) and half the per-group FMAs off the
// stream loop.
constexpr int kSumRow = 20;  // LDS floats per tile row of a chunk's group sums: 16 groups + pad

typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));  // RNE
}

// Three bf16 planes of eight fp32 values: plane p is the remainder left by
// planes 0..p-1 rounded to bf16 (each remainder is exact in fp32).
__device__ __forceinline__ void split3_bf16(const float (&v)[8], uint4 (&pl)[3]) {
  float r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = v[i];
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w[j] = bf16_pair(r[2 * j], r[2 * j + 1]);
      r[2 * j] -= __uint_as_float(w[j] << 16);
      r[2 * j + 1] -= __uint_as_float(w[j] & 0xFFFF0000u);
    }
    pl[p] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Eight bf16 scales times -128: exact (a power-of-two multiple of a bf16
// value is one), except past the bf16 range, where fp32 b - 128 s overflows too.
__device__ __forceinline__ uint4 times_m128(uint4 s) {
  const uint32_t w[4] = {s.x, s.y, s.z, s.w};
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    o[j] = bf16_pair(-128.0f * __uint_as_float(w[j] << 16), -128.0f * __uint_as_float(w[j] & 0xFFFF0000u));
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// The chunk correction for one row block: acc += A x b + A x (-128 s) over the
// 16 groups of the chunk.  sums: this lane's row of the chunk's group sums
// (groups 8 hh .. 8 hh + 7 at sums[0..7]); nvalid: how many of those 8 groups
// exist (a partial last chunk; a multiple of 4), the rest count as zero.
__device__ __forceinline__ void chunk_bias_mfma(f32x16_t& acc, const float* sums, uint4 bb, uint4 bs, int nvalid) {
  const float4 v0 = *reinterpret_cast<const float4*>(sums);
  const float4 v1 = *reinterpret_cast<const float4*>(sums + 4);
  float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  if (nvalid < 8) {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = j < nvalid ? v[j] : 0.0f;
  }
  uint4 pl[3];
  split3_bf16(v, pl);
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    acc = mfma_bf16(pl[p], bb, acc);
    acc = mfma_bf16(pl[p], bs, acc);
  }
}

// The chunk's B operands from LDS-staged scale rows (row: this column's
// bf16 scales or biases, G + 4 per row; groups g0 .. g0 + 7): 4-group pieces
// at or past G read as zero and are not read.
__device__ __forceinline__ uint4 sbl_groups8(const uint16_t* row, int g0, int G) {
  const uint2 z = make_uint2(0u, 0u);
  const uint2 p0 = g0 < G ? *reinterpret_cast<const uint2*>(row + g0) : z;
  const uint2 p1 = g0 + 4 < G ? *reinterpret_cast<const uint2*>(row + g0 + 4) : z;
  return make_uint4(p0.x, p0.y, p1.x, p1.y);
}

__device__ __forceinline__ Chunk16 load_chunk16(const uint16_t* S, const uint16_t* B, size_t off) {
  Chunk16 c;
  c.s0 = *reinterpret_cast<const uint4*>(S + off);
  c.s1 = *reinterpret_cast<const uint4*>(S + off + 8);
  c.b0 = *reinterpret_cast<const uint4*>(B + off);
  c.b1 = *reinterpret_cast<const uint4*>(B + off + 8);
  return c;
}

// bf16 element j (compile-time after unrolling) of 16 packed in two uint4
__device__ __forceinline__ float chunk_elem(const uint4& lo, const uint4& hi, int j) {
  const uint4& v = j < 8 ? lo : hi;
  const int d = (j & 7) >> 1;
  const uint32_t w = d == 0 ? v.x : (d == 1 ? v.y : (d == 2 ? v.z : v.w));
  return (j & 1) ? bf16_hi_to_f32(w) : bf16_lo_to_f32(w);
}

// bf16 element q (compile-time after unrolling) of 4 packed in two words
__device__ __forceinline__ float sb4_elem(uint32_t w01, uint32_t w23, int q) {
  const uint32_t w = q < 2 ? w01 : w23;
  return (q & 1) ? bf16_hi_to_f32(w) : bf16_lo_to_f32(w);
}

struct Codes4 {
  uint4 q[4];  // this lane's half (4 words) of each of 4 consecutive groups
};

__device__ __forceinline__ Codes4 load_codes4(const uint32_t* W, size_t rowc, int g0, int hh) {
  Codes4 c;
#pragma unroll
  for (int q = 0; q < 4; ++q) c.q[q] = *reinterpret_cast<const uint4*>(W + rowc + 8 * (g0 + q) + 4 * hh);
  return c;
}

// mxfp4 banks (E2M1 codes in the same word layout, one E8M0 scale byte per
// 32 inputs of a row).  The scale bytes of 4 consecutive 64-input groups of
// one row: byte 2 q + hh is the 32-input block of lane half hh in group q.
__device__ __forceinline__ uint2 load_mx_scales(const unsigned char* S, size_t rowb, int g0) {
  return *reinterpret_cast<const uint2*>(S + rowb + 2 * g0);
}

__device__ __forceinline__ uint32_t mx_scale_byte(uint2 s, int q, int hh) {
  return ((q < 2 ? s.x : s.y) >> (8 * (2 * (q & 1) + hh))) & 0xFFu;
}

// Exponent bytes for which every E2M1 magnitude (0.5 to 6) times 2^(e - 127)
// is a normal, finite bf16: there the scaled conversion is exact and the
// scale can be folded into the MFMA operand.  (The conversion takes only the
// exponent field of its f32 scale operand, which is all an E8M0 scale has.)
__device__ __forceinline__ bool mx_fold_exact(uint32_t e) { return e >= 2u && e <= 252u; }

// One code word (8 E2M1 codes, low nibble first) as 8 bf16 in element order,
// each multiplied by `sc` in the conversion.
__device__ __forceinline__ uint4 mx_word_bf16(uint32_t w, float sc) {
  return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3)));
}

// mxfp8: exponent bytes for which every nonzero E4M3 magnitude (2^-9 to 448)
// times 2^(e - 127) is a normal, finite bf16.
__device__ __forceinline__ bool mx8_fold_exact(uint32_t e) { return e >= 10u && e <= 246u; }

// Two code words of 8-bit E4M3 codes (lowest byte first) as 8 bf16 in element
// order, each multiplied by `sc` in the conversion.
__device__ __forceinline__ uint4 mx8_words_bf16(uint32_t w0, uint32_t w1, float sc) {
  return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, true)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, true)));
}

// The 4 MFMA B operands of group q: fp4, one code word each (Codes4 c holds
// the lane's 4 words of each group); fp8, two words each (c the first 4
// words of each group, c2 the last 4).
template <bool F8>
__device__ __forceinline__ void mx_group_operands(const Codes4& c, const Codes4& c2, int q, float sc, uint4 (&bq)[4]) {
  if constexpr (F8) {
    bq[0] = mx8_words_bf16(c.q[q].x, c.q[q].y, sc);
    bq[1] = mx8_words_bf16(c.q[q].z, c.q[q].w, sc);
    bq[2] = mx8_words_bf16(c2.q[q].x, c2.q[q].y, sc);
    bq[3] = mx8_words_bf16(c2.q[q].z, c2.q[q].w, sc);
  } else {
    bq[0] = mx_word_bf16(c.q[q].x, sc);
    bq[1] = mx_word_bf16(c.q[q].y, sc);
    bq[2] = mx_word_bf16(c.q[q].z, sc);
    bq[3] = mx_word_bf16(c.q[q].w, sc);
  }
}

// 8-bit codes: words 4 * part .. 4 * part + 3 of the lane half's 8 words in
// each of 4 consecutive groups (a group of one row is 16 words).
__device__ __forceinline__ Codes4 load_codes8(const uint32_t* W, size_t rowc, int g0, int hh, int part) {
  Codes4 c;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    c.q[q] = *reinterpret_cast<const uint4*>(W + rowc + 16 * (g0 + q) + 8 * hh + 4 * part);
  return c;
}

// The exact form of one 64-input mxfp4 group for one row block: acc += A x B
// with A = NPL staged planes of the rows (element order) and B = bq, the
// lane's 4 code words converted with unit scale.  Each 32-input block gets
// its own MFMA chain (the A operand of the other lane half zeroed) and is
// scaled in fp32 afterwards by s0 (inputs 0..31) or s1 (32..63), which also
// carries NaN (e = 255), subnormal and overflowing scales.
template <int NPL>
__device__ __forceinline__ void mx_mfma_split(f32x16_t& acc, const uint4 (&bq)[4], const unsigned char* const (&ap)[NPL],
                                              float s0, float s1, int hh) {
  const uint4 z = make_uint4(0u, 0u, 0u, 0u);
  f32x16_t p0 = {}, p1 = {};
#pragma unroll
  for (int pl = 0; pl < NPL; ++pl)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 av = *reinterpret_cast<const uint4*>(ap[pl] + 16 * s);
      // the product over one 32-input block: the other lane half's A operand is zeroed
      p0 = mfma_bf16(hh ? z : av, bq[s], p0);
      p1 = mfma_bf16(hh ? av : z, bq[s], p1);
    }
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = fmaf(s1, p1[i], fmaf(s0, p0[i], acc[i]));
  __builtin_amdgcn_sched_barrier(0);  // one row block at a time: no operand reads hoisted across blocks
}

// The block scales of one group for the lane's column from the lane's own
// exponent byte e and its partner half's: s0 for inputs 0..31, s1 for 32..63
// (2^(e - 127), NaN for e = 255).
__device__ __forceinline__ void mx_group_scales(uint32_t e, int hh, float& s0, float& s1) {
  const float own = mx_scaled(1.0f, e);
  const float oth = __shfl_xor(own, 32);
  s0 = hh ? oth : own;
  s1 = hh ? own : oth;
}

// Runs f(std::integral_constant<int, n>) with n = min(nrt, MT): the stream
// loops get the tile's count of 32-row blocks as a constant, so the MFMAs of
// all its blocks form one branch-free sequence whose LDS operand reads the
// compiler can overlap with the matrix work of the other blocks.
template <int MT, class F>
__device__ __forceinline__ void with_row_blocks(int nrt, F&& f) {
  if constexpr (MT == 1) {
    f(std::integral_constant<int, 1>{});
  } else {
    if (nrt >= MT) f(std::integral_constant<int, MT>{});
    else with_row_blocks<MT - 1>(nrt, f);
  }
}

// Kernel modes of the streaming kernels.  mxfp4 runs in two passes:
// kSortMxFold folds every block scale into the conversions (the fast form,
// exact while every exponent byte of the block's groups passes
// mx_fold_exact) and flags blocks where one does not; kSortMxExact then
// recomputes only the flagged blocks with per-32-input chains and fp32
// scaling, and returns at once elsewhere.
constexpr int kSortAffine = 0, kSortMxFold = 1, kSortMxExact = 2;
// kSortAffineSbl: affine, with the workgroup's scales and biases for the
// whole reduction read once into LDS at its start (one coalesced read of
// contiguous rows) instead of 16-group chunks along the stream, whose
// 128-byte lines had left L2 between chunks and were fetched again (1.35 x
// the algorithmic bytes).  Used where the LDS holds them, for tiles of two or
// more row blocks (down at T = 2048: 7-10 % faster; with one row block the
// read ahead of the stream cost more than the refetches, T = 512: 6 %
// slower) and for every width that is not a multiple of 1024 (the chunk
// loads need whole chunks).
constexpr int kSortAffineSbl = 3;
// mxfp8 (E4M3 codes, one byte per input; E8M0 scale per 32 inputs): the same
// two passes.
constexpr int kSortMx8Fold = 5, kSortMx8Exact = 6;
constexpr bool sort_mode_fold(int m) { return m == kSortMxFold || m == kSortMx8Fold; }
constexpr bool sort_mode_exact(int m) { return m == kSortMxExact || m == kSortMx8Exact; }
constexpr bool sort_mode_mx(int m) { return sort_mode_fold(m) || sort_mode_exact(m); }
constexpr bool sort_mode_f8(int m) { return m == kSortMx8Fold || m == kSortMx8Exact; }

// Copies rows [c0, c0 + ncols) of NAR scale / bias arrays (bf16 [.., G] per
// row, row c of expert e at (e * N + c) * G; G a multiple of 4) into LDS rows
// of G + 4 elements (the pad spreads a column group's reads over the banks);
// rows at or past N are skipped.  The global reads are PIECE-group pieces of
// contiguous rows (8 groups, 16 bytes, when G allows it, else 4), four per
// thread in flight at a time.
template <int NTHREADS, int NAR, int PIECE>
__device__ __forceinline__ void stage_scale_rows_p(uint16_t* dst, const uint16_t* const (&src)[NAR], int e, int N,
                                                   int c0, int ncols, int G, int tid) {
  typedef typename std::conditional<PIECE == 8, uint4, uint2>::type V;
  const int per_row = G / PIECE, GS = G + 4;
  const int total = NAR * ncols * per_row;
  for (int base = tid; base < total; base += 4 * NTHREADS) {
    V v[4];
    int to[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = base + u * NTHREADS;
      to[u] = -1;
      if (idx < total) {
        const int arr = idx / (ncols * per_row), rem = idx % (ncols * per_row);
        const int cl = rem / per_row, j = rem % per_row;
        if (c0 + cl < N) {
          v[u] = *reinterpret_cast<const V*>(src[arr] + ((size_t)e * N + c0 + cl) * G + PIECE * j);
          to[u] = (arr * ncols + cl) * GS + PIECE * j;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (to[u] < 0) continue;
      if constexpr (PIECE == 8) {  // rows of G + 4 elements are 8-byte aligned, not 16
        *reinterpret_cast<uint2*>(dst + to[u]) = make_uint2(v[u].x, v[u].y);
        *reinterpret_cast<uint2*>(dst + to[u] + 4) = make_uint2(v[u].z, v[u].w);
      } else {
        *reinterpret_cast<uint2*>(dst + to[u]) = v[u];
      }
    }
  }
}

template <int NTHREADS, int NAR>
__device__ __forceinline__ void stage_scale_rows(uint16_t* dst, const uint16_t* const (&src)[NAR], int e, int N,
                                                 int c0, int ncols, int G, int tid) {
  if (G % 8 == 0)
    stage_scale_rows_p<NTHREADS, NAR, 8>(dst, src, e, N, c0, ncols, G, tid);
  else
    stage_scale_rows_p<NTHREADS, NAR, 4>(dst, src, e, N, c0, ncols, G, tid);
}

// One iteration (4 groups of 64 inputs) of an mxfp4 column wave: acc[m] +=
// rows of block m (NPL planes `plane` bytes apart, from `arows`) x this
// lane's codes `cur` with exponent bytes `sc`, for the row blocks m < NRT
// and m < nrt (NRT a compile-time count, or MT with the run-time nrt).
template <int MT, int NRT, int MXM, int NPL>
__device__ __forceinline__ void mx_iteration(f32x16_t (&acc)[MT], const Codes4& cur, const Codes4& cur2, uint2 sc,
                                             const unsigned char* arows, size_t plane, int nrt, int hh,
                                             int& blk_split) {
  constexpr bool F8 = sort_mode_f8(MXM);
  if constexpr (sort_mode_fold(MXM)) {
    bool ok = true;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t e = mx_scale_byte(sc, q, hh);
      ok = ok && (F8 ? mx8_fold_exact(e) : mx_fold_exact(e));
    }
    if (!ok) blk_split = 1;  // the exact pass recomputes this block
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float fs = __uint_as_float(mx_scale_byte(sc, q, hh) << 23);  // 2^(e - 127) for 1 <= e <= 254
      uint4 bq[4];
      mx_group_operands<F8>(cur, cur2, q, fs, bq);
      if constexpr (NPL == 2) {
        // two planes (h hi and lo): one row block at a time, so the operands
        // of both planes stay few
#pragma unroll
        for (int m = 0; m < NRT; ++m) {
          if (m < nrt) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
              for (int pl = 0; pl < NPL; ++pl)
                acc[m] = mfma_bf16(*reinterpret_cast<const uint4*>(arows + (size_t)m * kRowTile * kV2Row +
                                                                   pl * plane + 128 * q + 16 * s),
                                   bq[s], acc[m]);
          }
        }
        continue;
      }
#pragma unroll
      for (int pl = 0; pl < NPL; ++pl) {
        // the group's operand reads first, then the MFMAs with the row
        // blocks interleaved (consecutive MFMAs write different accumulators)
        uint4 av[NRT][4];
#pragma unroll
        for (int m = 0; m < NRT; ++m)
#pragma unroll
          for (int s = 0; s < 4; ++s)
            av[m][s] = *reinterpret_cast<const uint4*>(arows + (size_t)m * kRowTile * kV2Row + pl * plane + 128 * q +
                                                       16 * s);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int m = 0; m < NRT; ++m) acc[m] = mfma_bf16(av[m][s], bq[s], acc[m]);
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float s0, s1;
      mx_group_scales(mx_scale_byte(sc, q, hh), hh, s0, s1);
      uint4 bq[4];
      mx_group_operands<F8>(cur, cur2, q, 1.0f, bq);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < NRT && m < nrt) {
          const unsigned char* const r = arows + (size_t)m * kRowTile * kV2Row + 128 * q;
          const unsigned char* ap[NPL];
#pragma unroll
          for (int pl = 0; pl < NPL; ++pl) ap[pl] = r + pl * plane;
          mx_mfma_split<NPL>(acc[m], bq, ap, s0, s1, hh);
        }
      }
    }
  }
}

// TAIL: the width is not a multiple of 1024, so the last chunk of 4
// iterations is partial (a compile-time switch: the check in the unrolled
// loop slowed the whole-chunk kernels by 5-8 %).
template <int MT, int MXM, bool TAIL>
__global__ __launch_bounds__(kV2Threads, 1) void k_sorted_gateup2(SortedArgs a) {
  constexpr bool MX = sort_mode_mx(MXM), SBL = MXM == kSortAffineSbl, F8 = sort_mode_f8(MXM);
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int blk_split;  // kSortMxFold: some group of this block needs the exact pass
  const int H = a.H, I = a.I, G = H / 64;
  // iterations of 4 groups (the width is a multiple of 256), in chunks of
  // 4; the chunked scale loads run only when the chunks are whole (width a
  // multiple of 1024)
  const int nit = G / 4, nch = (nit + 3) / 4;
  const int ncb = (I + kV2GuCols - 1) / kV2GuCols;
  int tile, cb;
  tile_of_block(ncb, tile, cb);
  if (tile >= (int)a.hdr[3]) return;
  if (sort_mode_exact(MXM) && a.mxflag_gu[blockIdx.x] == 0) return;
  const int4 td = a.tiles[tile];
  const int e = td.x, r0 = td.y, nrows = td.z;
  const int nrt = (nrows + kRowTile - 1) / kRowTile;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, hh = lane >> 5, lc = lane & 31;
  const int mat = wid >> 2, cw = wid & 3;
  const int col0 = cb * kV2GuCols + 32 * cw;
  const bool wave_on = col0 < I;
  const int col = wave_on ? col0 + lc : 0;

  constexpr int kRows = MT * kRowTile;
  // two staging buffers: iteration it reads buffer it & 1 while the rows of
  // it + 1 are written to the other, so one barrier per iteration suffices
  unsigned char* abuf0 = smem;                                              // [2][kRows][kV2Row]
  // affine: the group sums of the tile's rows for the 16 groups of a chunk,
  // [2 chunks][kRows][kSumRow] (chunk c in buffer c & 1)
  float* sums0 = reinterpret_cast<float*>(smem + 2 * kRows * kV2Row);
  int32_t* tok = reinterpret_cast<int32_t*>(sums0 + (MX ? 0 : 2 * kRows * kSumRow));  // [kRows]
  // kSortAffineSbl: [sg, bg, su, bu][128 columns][G + 4] bf16
  uint16_t* sbl = reinterpret_cast<uint16_t*>(tok + kRows);
  for (int r = tid; r < kRows; r += kV2Threads) tok[r] = a.perm[r0 + min(r, nrows - 1)] / a.k;
  if (tid == 0) blk_split = 0;
  __syncthreads();

  constexpr int kPer = kRows * 32 / kV2Threads;  // uint4 of x per thread and iteration
  uint4 st[kPer];
  float sst = 0.0f;
  auto stage_load = [&](int it) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int idx = tid + kV2Threads * j, r = idx >> 5, w = idx & 31;
      st[j] = *reinterpret_cast<const uint4*>(a.x + (size_t)tok[r] * H + 256 * it + 8 * w);
    }
    if constexpr (!MX) {
      const int si = min(tid, 4 * kRows - 1), q = si / kRows, r = si % kRows;
      sst = a.asum[(size_t)tok[r] * G + 4 * it + q];
    }
  };
  auto stage_store = [&](int buf, int itn) {
    unsigned char* abuf = abuf0 + (size_t)buf * kRows * kV2Row;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int idx = tid + kV2Threads * j, r = idx >> 5, w = idx & 31;
      // affine codes unpack in nibble-pair order, E2M1 conversions in element order
      *reinterpret_cast<uint4*>(abuf + (size_t)r * kV2Row + 16 * w) = MX ? st[j] : pair_activations(st[j]);
    }
    if (!MX && tid < 4 * kRows)  // group 4 itn + q of row r, q = tid / kRows, r = tid % kRows
      sums0[((itn >> 2) & 1) * kRows * kSumRow + (tid % kRows) * kSumRow + 4 * (itn & 3) + tid / kRows] = sst;
  };

  const uint32_t* W = mat ? a.wu : a.wg;
  const uint16_t* S = mat ? a.su : a.sg;
  const uint16_t* B = mat ? a.bu : a.bg;
  const size_t rowc = ((size_t)e * I + col) * (size_t)(H / (F8 ? 4 : 8));
  const size_t rows = ((size_t)e * I + col) * (size_t)G;
  const unsigned char* MS = reinterpret_cast<const unsigned char*>(S);  // mxfp4: E8M0 bytes [E][I][H / 32]
  const size_t rowb = ((size_t)e * I + col) * (size_t)(H / 32);

  f32x16_t acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[m][i] = 0.0f;

  // codes stay two iterations ahead; with PAIR they are requested two
  // iterations at a time (even iterations load it + 2 and it + 3 back to
  // back), so the two 128-byte pieces of a weight row reach HBM together.
  // Measured: faster for 2 and 3 row blocks (and mxfp4 gate/up with one),
  // slower for the other single-block kernels and past the registers of 4.
  constexpr bool PAIR = !F8 && ((MT == 2 || MT == 3) || (MXM == kSortMxFold && MT == 1));
  // mxfp8: cur and nx hold the two halves of one iteration's 8-bit codes,
  // loaded one iteration ahead (the same registers as two 4-bit iterations)
  Codes4 cur = F8 ? load_codes8(W, rowc, 0, hh, 0) : load_codes4(W, rowc, 0, hh);
  Codes4 nx = F8 ? load_codes8(W, rowc, 0, hh, 1) : load_codes4(W, rowc, 4 * min(1, nit - 1), hh);
  Codes4 pend;
  Chunk16 ch{};
  uint2 mcur{}, mnx{};
  if constexpr (MX) {
    mcur = load_mx_scales(MS, rowb, 0);
    mnx = load_mx_scales(MS, rowb, 4 * min(1, nit - 1));
  } else if constexpr (!SBL) {
    ch = load_chunk16(S, B, rows);
  }
  stage_load(0);
  if constexpr (SBL) {  // after the first code and row requests, so its wait overlaps theirs
    const uint16_t* const arrs[4] = {a.sg, a.bg, a.su, a.bu};
    stage_scale_rows<kV2Threads, 4>(sbl, arrs, e, I, cb * kV2GuCols, kV2GuCols, G, tid);
  }
  stage_store(0, 0);
  __syncthreads();

  for (int c = 0; c < nch; ++c) {
    Chunk16 chn;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int it = 4 * c + ii;
      if (TAIL && it >= nit) break;  // uniform over the workgroup
      const unsigned char* abuf = abuf0 + (size_t)(ii & 1) * kRows * kV2Row;  // it & 1
      stage_load(min(it + 1, nit - 1));
      Codes4 nn;
      if (F8) {
        nn = load_codes8(W, rowc, 4 * min(it + 1, nit - 1), hh, 0);
        pend = load_codes8(W, rowc, 4 * min(it + 1, nit - 1), hh, 1);
      } else if (!PAIR || (ii & 1) == 0) {  // ii is a compile-time value after unrolling
        nn = load_codes4(W, rowc, 4 * min(it + 2, nit - 1), hh);
        if (PAIR) pend = load_codes4(W, rowc, 4 * min(it + 3, nit - 1), hh);
      } else {
        nn = pend;
      }
      uint2 mnn{};
      if constexpr (MX) mnn = load_mx_scales(MS, rowb, 4 * min(it + 2, nit - 1));
      else if (!SBL && ii == 0) chn = load_chunk16(S, B, rows + 16 * min(c + 1, nch - 1));
      if (MX && wave_on) {
        const unsigned char* const arows = abuf + (size_t)lc * kV2Row + 64 * hh;
        with_row_blocks<MT>(nrt, [&](auto nrt_c) {
          constexpr int NRT = decltype(nrt_c)::value;
          mx_iteration<MT, NRT, MXM, 1>(acc, cur, nx, mcur, arows, 0, NRT, hh, blk_split);
        });
      } else if (!MX && wave_on) {
        uint2 sv{};  // kSortAffineSbl: this column's 4 scales of the iteration
        if constexpr (SBL) sv = *reinterpret_cast<const uint2*>(sbl + (size_t)(2 * mat * kV2GuCols + 32 * cw + lc) * (G + 4) + 4 * it);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t w4[4] = {cur.q[q].x, cur.q[q].y, cur.q[q].z, cur.q[q].w};
          uint4 bq[4];
#pragma unroll
          for (int s = 0; s < 4; ++s) bq[s] = unpack_codes(w4[s]);
          const float sc = SBL ? sb4_elem(sv.x, sv.y, q) : chunk_elem(ch.s0, ch.s1, 4 * ii + q);
          // the first two operand pieces of each row block are read during the
          // previous block's matrix chain (row blocks are tested at run time)
          const unsigned char* arow0 = abuf + (size_t)lc * kV2Row + 128 * q + 64 * hh;
          uint4 an0 = *reinterpret_cast<const uint4*>(arow0), an1 = *reinterpret_cast<const uint4*>(arow0 + 16);
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            if (m < nrt) {
              const unsigned char* arow = arow0 + (size_t)m * kRowTile * kV2Row;
              f32x16_t p = mfma_bf16(an0, bq[0], f32x16_t{});
              p = mfma_bf16(an1, bq[1], p);
              const uint4 a2 = *reinterpret_cast<const uint4*>(arow + 32), a3 = *reinterpret_cast<const uint4*>(arow + 48);
              if (m + 1 < MT) {  // unconditional at run time: every row of the tile is staged
                an0 = *reinterpret_cast<const uint4*>(arow + (size_t)kRowTile * kV2Row);
                an1 = *reinterpret_cast<const uint4*>(arow + (size_t)kRowTile * kV2Row + 16);
              }
              p = mfma_bf16(a2, bq[2], p);
              p = mfma_bf16(a3, bq[3], p);
#pragma unroll
              for (int i = 0; i < 16; ++i) acc[m][i] = fmaf(sc, p[i], acc[m][i]);  // (b - 128 s) A: per chunk
            }
          }
        }
      }
      stage_store((ii + 1) & 1, min(it + 1, nit - 1));
      __syncthreads();
      if (F8) {
        cur = nn;
        nx = pend;
      } else {
        cur = nx;
        nx = nn;
      }
      mcur = mnx;
      mnx = mnn;
    }
    // the chunk's (b - 128 s) A half of the correction (its group sums are
    // all staged: the last one landed before the barrier above)
    if (!MX && wave_on) {
      const int g0 = 16 * c + 8 * hh;
      uint4 bs, bb;
      if constexpr (SBL) {
        const uint16_t* srow_s = sbl + (size_t)(2 * mat * kV2GuCols + 32 * cw + lc) * (G + 4);
        bs = sbl_groups8(srow_s, g0, G);
        bb = sbl_groups8(srow_s + (size_t)kV2GuCols * (G + 4), g0, G);
      } else {
        bs = hh ? ch.s1 : ch.s0;
        bb = hh ? ch.b1 : ch.b0;
      }
      bs = times_m128(bs);
      const int nvalid = min(8, max(0, G - g0));
      const float* srow = sums0 + (c & 1) * kRows * kSumRow + 8 * hh;
#pragma unroll
      for (int m = 0; m < MT; ++m)
        if (m < nrt) chunk_bias_mfma(acc[m], srow + (m * kRowTile + lc) * kSumRow, bb, bs, nvalid);
    }
    ch = chn;
  }

  // up waves hand their sums to the gate waves through LDS (the staging area is free now)
  float* xch = reinterpret_cast<float*>(smem);  // [kRows][128]
  if (mat == 1 && wave_on) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
      if (m < nrt)
#pragma unroll
        for (int i = 0; i < 16; ++i) xch[(m * kRowTile + c_row(i, hh)) * kV2GuCols + 32 * cw + lc] = acc[m][i];
  }
  __syncthreads();
  if (sort_mode_fold(MXM) && tid == 0) a.mxflag_gu[blockIdx.x] = blk_split;
  if (mat == 1 || !wave_on) return;
  // affine: h columns in the down codes' nibble-pair order; mxfp4: element order
  const int scol = MX ? col : ((col & ~7) | ((col & 7) >> 1) | ((col & 1) << 2));
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m < nrt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = m * kRowTile + c_row(i, hh);
        const float gv = acc[m][i];
        const float uv = xch[r * kV2GuCols + 32 * cw + lc];
        const float hv = __builtin_amdgcn_ldexpf(gv / (1.0f + __expf(-gv)) * uv, -a.texp[tok[r]]);
        const uint32_t hi = f32_to_bf16_rne(hv);
        const float hif = __uint_as_float(hi << 16);
        const uint32_t lo = f32_to_bf16_rne(hv - hif);
        const float v = MX ? 0.0f : group_sum<32>(hif + __uint_as_float(lo << 16));
        if (r < nrows) {
          const size_t o = (size_t)(r0 + r) * I;
          a.hhi[o + scol] = (uint16_t)hi;
          a.hlo[o + scol] = (uint16_t)lo;
          if (!MX && lc == 0) a.hsum2[(size_t)(r0 + r) * (I / 32) + col0 / 32] = v;
        }
      }
    }
  }
}

// staging buffers of the down streaming kernel: two while they fit the LDS
constexpr int down2_buffers(int mt) {
  return (size_t)2 * 2 * mt * kRowTile * kV2Row + (size_t)2 * mt * kRowTile * kSumRow * 4 <= 160 * 1024 ? 2 : 1;
}

template <int MT, int MXM, bool TAIL>
__global__ __launch_bounds__(kV2Threads, 1) void k_sorted_down2(SortedArgs a) {
  constexpr bool MX = sort_mode_mx(MXM), SBL = MXM == kSortAffineSbl, F8 = sort_mode_f8(MXM);
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int blk_split;  // kSortMxFold: some group of this block needs the exact pass
  const int H = a.H, I = a.I, G = I / 64;
  // iterations of 4 groups (the width is a multiple of 256), in chunks of
  // 4; the chunked scale loads run only when the chunks are whole (width a
  // multiple of 1024)
  const int nit = G / 4, nch = (nit + 3) / 4;
  const int ncb = (H + kV2DnCols - 1) / kV2DnCols;
  int tile, cb;
  tile_of_block(ncb, tile, cb);
  if (tile >= (int)a.hdr[3]) return;
  if (sort_mode_exact(MXM) && a.mxflag_dn[blockIdx.x] == 0) return;
  if (threadIdx.x == 0) blk_split = 0;  // published by the first barrier of the stream loop
  const int4 td = a.tiles[tile];
  const int e = td.x, r0 = td.y, nrows = td.z;
  const int nrt = (nrows + kRowTile - 1) / kRowTile;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, hh = lane >> 5, lc = lane & 31;
  const int col0 = cb * kV2DnCols + 32 * wid;
  const bool wave_on = col0 < H;
  const int col = wave_on ? col0 + lc : 0;

  constexpr int kRows = MT * kRowTile;
  // two staging buffers when they fit the LDS (one barrier per iteration),
  // else one (a second barrier before the rows of the next iteration land)
  constexpr int NB = down2_buffers(MT);
  unsigned char* abuf0 = smem;                                                     // [NB][2 planes][kRows][kV2Row]
  // affine: the group sums of the tile's rows for the 16 groups of a chunk,
  // [2 chunks][kRows][kSumRow] (chunk c in buffer c & 1)
  float* sums0 = reinterpret_cast<float*>(smem + (size_t)NB * 2 * kRows * kV2Row);
  // kSortAffineSbl: [sd, bd][256][G + 4]
  uint16_t* sbl = reinterpret_cast<uint16_t*>(sums0 + (MX ? 0 : 2 * kRows * kSumRow));

  constexpr int kPer = kRows * 32 / kV2Threads;  // 16-byte pieces per thread, iteration and plane
  u32x4_t sth[kPer], stl[kPer];
  float sst = 0.0f;
  auto stage_load = [&](int it) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int idx = tid + kV2Threads * j, r = min(idx >> 5, nrows - 1), w = idx & 31;
      const size_t o = (size_t)(r0 + r) * I + 256 * it + 8 * w;
      sth[j] = *reinterpret_cast<const u32x4_t*>(a.hhi + o);
      stl[j] = *reinterpret_cast<const u32x4_t*>(a.hlo + o);
    }
    if constexpr (!MX) {
      const int si = min(tid, 4 * kRows - 1), q = si / kRows, r = min(si % kRows, nrows - 1);
      const float* hs = a.hsum2 + (size_t)(r0 + r) * (I / 32) + 2 * (4 * it + q);
      sst = hs[0] + hs[1];
    }
  };
  auto stage_store = [&](int buf, int itn) {
    unsigned char* abuf = abuf0 + (size_t)buf * 2 * kRows * kV2Row;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int idx = tid + kV2Threads * j, r = idx >> 5, w = idx & 31;
      *reinterpret_cast<u32x4_t*>(abuf + (size_t)r * kV2Row + 16 * w) = sth[j];
      *reinterpret_cast<u32x4_t*>(abuf + (size_t)(kRows + r) * kV2Row + 16 * w) = stl[j];
    }
    if (!MX && tid < 4 * kRows)  // group 4 itn + q of row r, q = tid / kRows, r = tid % kRows
      sums0[((itn >> 2) & 1) * kRows * kSumRow + (tid % kRows) * kSumRow + 4 * (itn & 3) + tid / kRows] = sst;
  };

  const size_t rowc = ((size_t)e * H + col) * (size_t)(I / (F8 ? 4 : 8));
  const size_t rows = ((size_t)e * H + col) * (size_t)G;
  const unsigned char* MS = reinterpret_cast<const unsigned char*>(a.sd);  // mxfp4: E8M0 bytes [E][H][I / 32]
  const size_t rowb = ((size_t)e * H + col) * (size_t)(I / 32);

  f32x16_t acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[m][i] = 0.0f;

  // codes stay two iterations ahead; with PAIR they are requested two
  // iterations at a time (even iterations load it + 2 and it + 3 back to
  // back), so the two 128-byte pieces of a weight row reach HBM together.
  // Measured: faster for 2 and 3 row blocks (and mxfp4 gate/up with one),
  // slower for the other single-block kernels and past the registers of 4.
  constexpr bool PAIR = MT == 2 || MT == 3;
  // mxfp8: cur and nx hold the two halves of one iteration's 8-bit codes,
  // loaded one iteration ahead (the same registers as two 4-bit iterations)
  Codes4 cur = F8 ? load_codes8(a.wd, rowc, 0, hh, 0) : load_codes4(a.wd, rowc, 0, hh);
  Codes4 nx = F8 ? load_codes8(a.wd, rowc, 0, hh, 1) : load_codes4(a.wd, rowc, 4 * min(1, nit - 1), hh);
  Codes4 pend;
  Chunk16 ch{};
  uint2 mcur{}, mnx{};
  if constexpr (MX) {
    mcur = load_mx_scales(MS, rowb, 0);
    mnx = load_mx_scales(MS, rowb, 4 * min(1, nit - 1));
  } else if constexpr (!SBL) {
    ch = load_chunk16(a.sd, a.bd, rows);
  }
  stage_load(0);
  if constexpr (SBL) {  // after the first code and row requests, so its wait overlaps theirs
    const uint16_t* const arrs[2] = {a.sd, a.bd};
    stage_scale_rows<kV2Threads, 2>(sbl, arrs, e, H, cb * kV2DnCols, kV2DnCols, G, tid);
  }
  stage_store(0, 0);
  __syncthreads();

  for (int c = 0; c < nch; ++c) {
    Chunk16 chn;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int it = 4 * c + ii;
      if (TAIL && it >= nit) break;  // uniform over the workgroup
      const int cbuf = NB == 2 ? (ii & 1) : 0;  // it & 1
      const unsigned char* abuf = abuf0 + (size_t)cbuf * 2 * kRows * kV2Row;
      stage_load(min(it + 1, nit - 1));
      Codes4 nn;
      if (F8) {
        nn = load_codes8(a.wd, rowc, 4 * min(it + 1, nit - 1), hh, 0);
        pend = load_codes8(a.wd, rowc, 4 * min(it + 1, nit - 1), hh, 1);
      } else if (!PAIR || (ii & 1) == 0) {  // ii is a compile-time value after unrolling
        nn = load_codes4(a.wd, rowc, 4 * min(it + 2, nit - 1), hh);
        if (PAIR) pend = load_codes4(a.wd, rowc, 4 * min(it + 3, nit - 1), hh);
      } else {
        nn = pend;
      }
      uint2 mnn{};
      if constexpr (MX) mnn = load_mx_scales(MS, rowb, 4 * min(it + 2, nit - 1));
      else if (!SBL && ii == 0) chn = load_chunk16(a.sd, a.bd, rows + 16 * min(c + 1, nch - 1));
      if (MX && wave_on) {
        const unsigned char* const arows = abuf + (size_t)lc * kV2Row + 64 * hh;
        // row blocks tested at run time: the two planes leave no registers
        // for a copy of the loop per row-block count
        mx_iteration<MT, MT, MXM, 2>(acc, cur, nx, mcur, arows, (size_t)kRows * kV2Row, nrt, hh, blk_split);
      } else if (!MX && wave_on) {
        uint2 sv{};  // kSortAffineSbl: this column's 4 scales of the iteration
        if constexpr (SBL) sv = *reinterpret_cast<const uint2*>(sbl + (size_t)(32 * wid + lc) * (G + 4) + 4 * it);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t w4[4] = {cur.q[q].x, cur.q[q].y, cur.q[q].z, cur.q[q].w};
          uint4 bq[4];
#pragma unroll
          for (int s = 0; s < 4; ++s) bq[s] = unpack_codes(w4[s]);
          const float sc = SBL ? sb4_elem(sv.x, sv.y, q) : chunk_elem(ch.s0, ch.s1, 4 * ii + q);
          // the first hi and lo operand pieces of each row block are read during
          // the previous block's matrix chain (row blocks are tested at run time)
          const unsigned char* ph0 = abuf + (size_t)lc * kV2Row + 128 * q + 64 * hh;
          uint4 anh = *reinterpret_cast<const uint4*>(ph0),
                anl = *reinterpret_cast<const uint4*>(ph0 + (size_t)kRows * kV2Row);
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            if (m < nrt) {
              const unsigned char* ph = ph0 + (size_t)m * kRowTile * kV2Row;
              const unsigned char* pl = ph + (size_t)kRows * kV2Row;
              f32x16_t p = mfma_bf16(anh, bq[0], f32x16_t{});
              p = mfma_bf16(anl, bq[0], p);
              if (m + 1 < MT) {  // unconditional at run time: every row of the tile is staged
                anh = *reinterpret_cast<const uint4*>(ph + (size_t)kRowTile * kV2Row);
                anl = *reinterpret_cast<const uint4*>(pl + (size_t)kRowTile * kV2Row);
              }
#pragma unroll
              for (int s = 1; s < 4; ++s) {
                p = mfma_bf16(*reinterpret_cast<const uint4*>(ph + 16 * s), bq[s], p);
                p = mfma_bf16(*reinterpret_cast<const uint4*>(pl + 16 * s), bq[s], p);
              }
#pragma unroll
              for (int i = 0; i < 16; ++i) acc[m][i] = fmaf(sc, p[i], acc[m][i]);  // (b - 128 s) A: per chunk
            }
          }
        }
      }
      if (NB == 1) __syncthreads();
      stage_store(NB == 2 ? ((ii + 1) & 1) : 0, min(it + 1, nit - 1));
      __syncthreads();
      if (F8) {
        cur = nn;
        nx = pend;
      } else {
        cur = nx;
        nx = nn;
      }
      mcur = mnx;
      mnx = mnn;
    }
    // the chunk's (b - 128 s) A half of the correction, A = sum of h hi + lo
    // over each group (all staged: the last one landed before the barrier above)
    if (!MX && wave_on) {
      const int g0 = 16 * c + 8 * hh;
      uint4 bs, bb;
      if constexpr (SBL) {
        const uint16_t* srow_s = sbl + (size_t)(32 * wid + lc) * (G + 4);
        bs = sbl_groups8(srow_s, g0, G);
        bb = sbl_groups8(srow_s + (size_t)kV2DnCols * (G + 4), g0, G);
      } else {
        bs = hh ? ch.s1 : ch.s0;
        bb = hh ? ch.b1 : ch.b0;
      }
      bs = times_m128(bs);
      const int nvalid = min(8, max(0, G - g0));
      const float* srow = sums0 + (c & 1) * kRows * kSumRow + 8 * hh;
#pragma unroll
      for (int m = 0; m < MT; ++m)
        if (m < nrt) chunk_bias_mfma(acc[m], srow + (m * kRowTile + lc) * kSumRow, bb, bs, nvalid);
    }
    ch = chn;
  }

  if (sort_mode_fold(MXM) && tid == 0) a.mxflag_dn[blockIdx.x] = blk_split;  // after the loop's last barrier
  if (!wave_on) return;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m < nrt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = m * kRowTile + c_row(i, hh);
        if (r < nrows) a.ys[(size_t)(r0 + r) * H + col] = acc[m][i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// combine
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_sorted_combine(SortedArgs a) {
  const int H = a.H, k = a.k, n4 = H >> 2;
  const int it = blockIdx.x * 256 + threadIdx.x;
  const int t = blockIdx.y;
  if (it >= n4) return;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int j = 0; j < k; ++j) {
    const int p = t * k + j;
    const int e = a.ids[p];
    if (e < 0 || e >= a.E) continue;
    const float w = a.tw[p];
    const float4 v = reinterpret_cast<const float4*>(a.ys + (size_t)a.inv[p] * H)[it];
    acc.x = fmaf(w, v.x, acc.x);
    acc.y = fmaf(w, v.y, acc.y);
    acc.z = fmaf(w, v.z, acc.z);
    acc.w = fmaf(w, v.w, acc.w);
  }
  // the pairs' outputs carry the token's 2^-e_t (see k_token_gsum)
  const int te = a.texp[t];
  acc.x = __builtin_amdgcn_ldexpf(acc.x, te);
  acc.y = __builtin_amdgcn_ldexpf(acc.y, te);
  acc.z = __builtin_amdgcn_ldexpf(acc.z, te);
  acc.w = __builtin_amdgcn_ldexpf(acc.w, te);
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

size_t r256(size_t v) { return (v + 255) & ~size_t(255); }

size_t sort_lds(int E) { return (size_t)4 * (E + 1 + 2 * kSortThreads); }
size_t gateup_lds(int mt) { return (size_t)2 * mt * kRowTile * kRowBytes + 3 * mt * kRowTile * 4; }
size_t down_lds(int mt) { return (size_t)4 * mt * kRowTile * kRowBytes + 2 * mt * kRowTile * 4; }

}  // namespace

int sorted_row_blocks(int T, int k, int E) {
  const double per = (double)T * k / (double)E;  // mean pairs per expert
  return per <= 24.0 ? 1 : (per <= 48.0 ? 2 : (per <= 72.0 ? 3 : 4));
}

int sorted_tiles_max(int T, int k, int E, int bm) {
  const long P = (long)T * k;
  return (int)(P / bm + (P < E ? P : E) + 1);
}

// Blocks of the larger of the two streaming grids (tiles rounded up to 8,
// times column blocks), for any row-block count.
size_t sorted_flag_count(int T, int k, int E, int H, int I) {
  // tiles of 32 rows: at least as many as any row-block count gives
  const size_t tiles8 = (size_t)(sorted_tiles_max(T, k, E, kRowTile) + 7) / 8 * 8;
  const int ngu = (I + kV2GuCols - 1) / kV2GuCols, ndn = (H + kV2DnCols - 1) / kV2DnCols;
  return tiles8 * (size_t)(ngu > ndn ? ngu : ndn);
}

SortedWorkspace sorted_workspace_layout(int T, int k, int E, int H, int I) {
  SortedWorkspace w{};
  const size_t P = (size_t)T * k;
  size_t off = 0;
  w.hdr = off;      off = r256(off + 256);
  w.offsets = off;  off = r256(off + (size_t)(E + 1) * 4);
  w.perm = off;     off = r256(off + P * 4);
  w.inv = off;      off = r256(off + P * 4);
  w.rank_tmp = off; off = r256(off + P * 4);
  w.tiles = off;    off = r256(off + (size_t)sorted_tiles_max(T, k, E, kRowTile) * 16);
  w.asum = off;     off = r256(off + (size_t)T * (H / 64) * 4);
  w.texp = off;     off = r256(off + (size_t)T * 4);
  w.hhi = off;      off = r256(off + P * I * 2);
  w.hlo = off;      off = r256(off + P * I * 2);
  w.hsum2 = off;    off = r256(off + P * (I / 32) * 4);
  w.ys = off;       off = r256(off + P * H * 4);
  // mxfp4: one flag per block of the streaming gate/up and down grids
  w.mxflag = off;   off = r256(off + (size_t)2 * sorted_flag_count(T, k, E, H, I) * 4);
  w.total = off;
  return w;
}

bool sorted_mx_shape_supported(int T, int k, int E, int H, int I) {
  return H % 256 == 0 && I % 256 == 0 && sorted_shape_supported(T, k, E, H, I);
}

bool sorted_shape_supported(int T, int k, int E, int H, int I) {
  (void)H; (void)I;
  const long P = (long)T * k;
  // T <= 65535: the combine grid's second dimension is the token
  return T <= 65535 && E <= MOE_Q4_MAX_E && P < (1L << 30) && sort_lds(E) <= 160 * 1024;
}

int sort_launch(const SortedArgs& a, hipStream_t stream) {
  const int P = a.T * a.k;
  hipLaunchKernelGGL(k_sort_scan, dim3(1), dim3(kSortThreads), sort_lds(a.E), stream, a);
  if (hipGetLastError() != hipSuccess) return MOE_Q4_ERR_LAUNCH;
  hipLaunchKernelGGL(k_sort_rank, dim3((P + 255) / 256), dim3(256), 0, stream, a);
  return hipGetLastError() == hipSuccess ? MOE_Q4_OK : MOE_Q4_ERR_LAUNCH;
}

// staged rows, the affine chunk sums (mx: none) and the row tokens (gate/up)
size_t gateup2_lds(int mt, bool mx) {
  return (size_t)2 * mt * kRowTile * kV2Row + (mx ? 0 : (size_t)2 * mt * kRowTile * kSumRow * 4) + mt * kRowTile * 4;
}
size_t down2_lds(int mt, bool mx) {
  return (size_t)down2_buffers(mt) * 2 * mt * kRowTile * kV2Row + (mx ? 0 : (size_t)2 * mt * kRowTile * kSumRow * 4);
}
// the same plus the workgroup's scale and bias rows (kSortAffineSbl)
size_t gateup2_sbl_lds(int mt, int H) { return gateup2_lds(mt, false) + (size_t)4 * kV2GuCols * (H / 64 + 4) * 2; }
size_t down2_sbl_lds(int mt, int I) { return down2_lds(mt, false) + (size_t)2 * kV2DnCols * (I / 64 + 4) * 2; }
constexpr size_t kSortLdsMax = 160 * 1024 - 256;  // the static __shared__ word and slack

// alignment the scale-row pieces of a width need: 16 bytes for 8-group pieces, else 8
bool aligned_for(int width, const void* p) { return ((uintptr_t)p & (width % 512 == 0 ? 15 : 7)) == 0; }

// The LDS-staged scales: widths that are multiples of 256 (a scale row is
// copied in pieces of 8 or 4 groups), where the LDS holds them and the
// arrays allow 16-byte (8 groups) or 8-byte reads; used for 2 or more row blocks (with one, the
// read ahead of the stream cost more than the refetches it saves) and for
// widths that are not multiples of 1024.
bool gateup2_sbl_fits(const SortedArgs& a, int mt) {
  return a.H % 256 == 0 && (mt >= 2 || a.H % 1024 != 0) && gateup2_sbl_lds(mt, a.H) <= kSortLdsMax &&
         aligned_for(a.H, a.sg) && aligned_for(a.H, a.bg) && aligned_for(a.H, a.su) && aligned_for(a.H, a.bu);
}
bool down2_sbl_fits(const SortedArgs& a, int mt) {
  return a.I % 256 == 0 && (mt >= 2 || a.I % 1024 != 0) && down2_sbl_lds(mt, a.I) <= kSortLdsMax &&
         aligned_for(a.I, a.sd) && aligned_for(a.I, a.bd);
}

// mxfp4 / mxfp8: the folded pass, then the exact pass over the blocks it flagged
template <int MT, bool TAIL, int FOLD, int EXACT>
int mx_launch(const SortedArgs& a, bool down, int tiles8, hipStream_t stream) {
  if (!down) {
    const int ncb = (a.I + kV2GuCols - 1) / kV2GuCols;
    hipLaunchKernelGGL((k_sorted_gateup2<MT, FOLD, TAIL>), dim3(tiles8 * ncb), dim3(kV2Threads), gateup2_lds(MT, true), stream,
                       a);
    if (hipGetLastError() != hipSuccess) return MOE_Q4_ERR_LAUNCH;
    hipLaunchKernelGGL((k_sorted_gateup2<MT, EXACT, TAIL>), dim3(tiles8 * ncb), dim3(kV2Threads), gateup2_lds(MT, true), stream,
                       a);
  } else {
    const int ncb = (a.H + kV2DnCols - 1) / kV2DnCols;
    hipLaunchKernelGGL((k_sorted_down2<MT, FOLD, TAIL>), dim3(tiles8 * ncb), dim3(kV2Threads), down2_lds(MT, true), stream, a);
    if (hipGetLastError() != hipSuccess) return MOE_Q4_ERR_LAUNCH;
    hipLaunchKernelGGL((k_sorted_down2<MT, EXACT, TAIL>), dim3(tiles8 * ncb), dim3(kV2Threads), down2_lds(MT, true), stream, a);
  }
  return hipGetLastError() == hipSuccess ? MOE_Q4_OK : MOE_Q4_ERR_LAUNCH;
}

template <int MT, bool TAIL>
int gemm_launch(const SortedArgs& a, bool down, hipStream_t stream) {
  const int tiles8 = (a.tiles_max + 7) / 8 * 8;
  if (a.fmt == kFmtMxfp4 || a.fmt == kFmtMxfp8) {
    // the streaming kernels only (H and I multiples of 256, checked by the caller)
    if (a.H % 256 || a.I % 256) return MOE_Q4_ERR_UNSUPPORTED;
    return a.fmt == kFmtMxfp8 ? mx_launch<MT, TAIL, kSortMx8Fold, kSortMx8Exact>(a, down, tiles8, stream)
                              : mx_launch<MT, TAIL, kSortMxFold, kSortMxExact>(a, down, tiles8, stream);
  } else if (!down && gateup2_sbl_fits(a, MT)) {
    // scales in LDS: tiles of 2 or more row blocks, and any width that is not
    // a multiple of 1024 (the chunked scale loads need whole chunks)
    const int ncb = (a.I + kV2GuCols - 1) / kV2GuCols;
    hipLaunchKernelGGL((k_sorted_gateup2<MT, kSortAffineSbl, TAIL>), dim3(tiles8 * ncb), dim3(kV2Threads),
                       gateup2_sbl_lds(MT, a.H), stream, a);
  } else if (!down && a.H % 1024 == 0) {
    const int ncb = (a.I + kV2GuCols - 1) / kV2GuCols;
    hipLaunchKernelGGL((k_sorted_gateup2<MT, kSortAffine, false>), dim3(tiles8 * ncb), dim3(kV2Threads), gateup2_lds(MT, false),
                       stream, a);
  } else if (down && down2_sbl_fits(a, MT)) {
    const int ncb = (a.H + kV2DnCols - 1) / kV2DnCols;
    hipLaunchKernelGGL((k_sorted_down2<MT, kSortAffineSbl, TAIL>), dim3(tiles8 * ncb), dim3(kV2Threads),
                       down2_sbl_lds(MT, a.I), stream, a);
  } else if (down && a.I % 1024 == 0) {
    const int ncb = (a.H + kV2DnCols - 1) / kV2DnCols;
    hipLaunchKernelGGL((k_sorted_down2<MT, kSortAffine, false>), dim3(tiles8 * ncb), dim3(kV2Threads), down2_lds(MT, false), stream,
                       a);
  } else if (!down) {
    const int ncb = (a.I + kGuCols - 1) / kGuCols;
    hipLaunchKernelGGL(k_sorted_gateup<MT>, dim3(tiles8 * ncb), dim3(kMmThreads), gateup_lds(MT), stream, a);
  } else {
    const int ncb = (a.H + kDnCols - 1) / kDnCols;
    hipLaunchKernelGGL(k_sorted_down<MT>, dim3(tiles8 * ncb), dim3(kMmThreads), down_lds(MT), stream, a);
  }
  return hipGetLastError() == hipSuccess ? MOE_Q4_OK : MOE_Q4_ERR_LAUNCH;
}

template <bool TAIL>
int gemm_dispatch_tail(const SortedArgs& a, bool down, hipStream_t stream) {
  switch (a.bm / kRowTile) {
    case 1: return gemm_launch<1, TAIL>(a, down, stream);
    case 2: return gemm_launch<2, TAIL>(a, down, stream);
    case 3: return gemm_launch<3, TAIL>(a, down, stream);
    case 4: return gemm_launch<4, TAIL>(a, down, stream);
    default: return MOE_Q4_ERR_UNSUPPORTED;
  }
}

int gemm_dispatch(const SortedArgs& a, bool down, hipStream_t stream) {
  // the streaming kernels' width: H for gate/up, I for down
  return ((down ? a.I : a.H) % 1024) ? gemm_dispatch_tail<true>(a, down, stream)
                                     : gemm_dispatch_tail<false>(a, down, stream);
}

int sorted_forward_launch(const SortedArgs& a, unsigned stages, hipStream_t stream) {
  if (stages & MOE_Q4_STAGE_GATEUP) {
    int st = sort_launch(a, stream);
    if (st) return st;
    // per-token exponents (every format) and activation group sums (affine)
    hipLaunchKernelGGL(k_token_gsum, dim3(a.T), dim3(256), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return MOE_Q4_ERR_LAUNCH;
    st = gemm_dispatch(a, false, stream);
    if (st) return st;
  }
  if (stages & MOE_Q4_STAGE_DOWN) {
    const int st = gemm_dispatch(a, true, stream);
    if (st) return st;
    hipLaunchKernelGGL(k_sorted_combine, dim3((a.H / 4 + 255) / 256, a.T), dim3(256), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return MOE_Q4_ERR_LAUNCH;
  }
  return MOE_Q4_OK;
}

}  // namespace moeq4
