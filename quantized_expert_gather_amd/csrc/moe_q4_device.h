// Device helpers of the union path (gfx950, wave64).  Internal header.
//
// Sources (web pages): the union of routed experts with one weight stream per
// distinct expert follows the mlx discussion "Small-L fused expert gather for
// fine-grained MoE decode" (implication 1 of the adjacent-token overlap
// section); the affine 4-bit, group-64 storage and the SwitchGLU order follow
// the mlx issue "gather_qmm at M=1 streams 4-bit expert weights at ~half the
// bandwidth of M=4" (section "Numbers", moe_bench script).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moeq4 {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Exponent bits of bf16 128.0 in both halves: OR-ing a 4-bit code q into the
// low mantissa bits of each half gives the bf16 pair (128 + q_lo, 128 + q_hi)
// exactly (bf16 has 7 mantissa bits; at exponent 2^7 one mantissa step is 1).
constexpr uint32_t kMagic128 = 0x43004300u;

// Splits one 32-bit word of eight codes (nibble c holds element c) into four
// bf16 pairs: out[kk] = (128 + q[kk], 128 + q[kk + 4]) in (low, high) halves.
__device__ __forceinline__ void unpack_word(uint32_t w, uint32_t out[4]) {
  out[0] = (w & 0x000F000Fu) | kMagic128;
  out[1] = ((w >> 4) & 0x000F000Fu) | kMagic128;
  out[2] = ((w >> 8) & 0x000F000Fu) | kMagic128;
  out[3] = ((w >> 12) & 0x000F000Fu) | kMagic128;
}

// acc + a.lo * b.lo + a.hi * b.hi with bf16 inputs and fp32 accumulation
// (v_dot2c_f32_bf16; bf16 x bf16 products are exact in fp32).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b),
                                         acc, false);
}

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// fp32 -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Reorders eight consecutive bf16 values e0..e7 (packed two per word, low
// half first) into the pairs that unpack_word produces for codes:
// (e0,e4), (e1,e5), (e2,e6), (e3,e7).
__device__ __forceinline__ uint4 pair_activations(uint4 v) {
  uint4 r;
  r.x = (v.x & 0xFFFFu) | (v.z << 16);
  r.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
  r.z = (v.y & 0xFFFFu) | (v.w << 16);
  r.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
  return r;
}

// Sum of eight bf16 values packed in a uint4, ascending element order.
__device__ __forceinline__ float sum8_bf16(uint4 v, float acc) {
  acc += bf16_lo_to_f32(v.x); acc += bf16_hi_to_f32(v.x);
  acc += bf16_lo_to_f32(v.y); acc += bf16_hi_to_f32(v.y);
  acc += bf16_lo_to_f32(v.z); acc += bf16_hi_to_f32(v.z);
  acc += bf16_lo_to_f32(v.w); acc += bf16_hi_to_f32(v.w);
  return acc;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the WIDTH lanes of an aligned lane group (WIDTH a power of two
// <= 64); every lane of the group receives the sum.  Within 16-lane rows the
// steps are DPP lane permutes (xor 1, xor 2, half-row mirror, row mirror);
// across rows they are lane shuffles.
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (WIDTH >= 2) v += dpp_f32<0xB1>(v);   // quad_perm(1,0,3,2)
  if constexpr (WIDTH >= 4) v += dpp_f32<0x4E>(v);   // quad_perm(2,3,0,1)
  if constexpr (WIDTH >= 8) v += dpp_f32<0x141>(v);  // row_half_mirror
  if constexpr (WIDTH >= 16) v += dpp_f32<0x140>(v); // row_mirror
  if constexpr (WIDTH >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (WIDTH >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave (all lanes active).
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
  return v;
}

// Index of the n-th set bit (n counted from 0) of m; m has more than n bits set.
__device__ __forceinline__ int nth_set_bit(uint32_t m, int n) {
  for (int c = 0; c < n; ++c) m &= m - 1u;
  return __builtin_ctz(m);
}

// Union of the routes, built in LDS by one workgroup.
//   bitmap[EW]  presence of each expert id      scan[EW]  exclusive popcount prefix
//   uniq[P]     distinct ids ascending          mask[P]   token mask per distinct id
//   off[P+1]    exclusive prefix of popcount(mask): first pair slot of each distinct id
//   scal[0] = u (distinct ids), scal[1] = 1 if an id fell outside [0, E)
struct UnionLds {
  uint32_t* bitmap;
  int32_t* scan;
  int32_t* uniq;
  uint32_t* mask;
  int32_t* off;
  int32_t* scal;
};

// Every thread of the workgroup must call this (it contains barriers).
// Requires blockDim.x >= 64, L <= 32, P = L * k.
__device__ inline void build_union(const int32_t* __restrict__ ids, int P, int k, int E, const UnionLds& s) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int EW = (E + 31) >> 5;
  for (int w = tid; w < EW; w += nthr) s.bitmap[w] = 0u;
  for (int i = tid; i < P; i += nthr) s.mask[i] = 0u;
  if (tid == 0) s.scal[1] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += nthr) {
    const int e = ids[p];
    if (e >= 0 && e < E)
      atomicOr(&s.bitmap[e >> 5], 1u << (e & 31));
    else
      s.scal[1] = 1;
  }
  __syncthreads();
  if (tid < 64) {
    int carry = 0;
    for (int base = 0; base < EW; base += 64) {
      const int w = base + tid;
      const int c = (w < EW) ? __popc(s.bitmap[w]) : 0;
      const int incl = wave_incl_scan(c);
      if (w < EW) s.scan[w] = carry + incl - c;
      carry += __shfl(incl, 63, 64);
    }
    if (tid == 0) s.scal[0] = carry;
  }
  __syncthreads();
  for (int p = tid; p < P; p += nthr) {
    const int e = ids[p];
    if (e >= 0 && e < E) {
      const uint32_t word = s.bitmap[e >> 5];
      const int r = s.scan[e >> 5] + __popc(word & ((1u << (e & 31)) - 1u));
      s.uniq[r] = e;  // every duplicate writes the same value
      atomicOr(&s.mask[r], 1u << (p / k));
    }
  }
  __syncthreads();
  const int u = s.scal[0];
  if (tid < 64) {
    int carry = 0;
    for (int base = 0; base < u; base += 64) {
      const int i = base + tid;
      const int c = (i < u) ? __popc(s.mask[i]) : 0;
      const int incl = wave_incl_scan(c);
      if (i < u) s.off[i] = carry + incl - c;
      carry += __shfl(incl, 63, 64);
    }
    if (tid == 0) s.off[u] = carry;
  }
  __syncthreads();
}

// Router weight of token t for expert e: the fp32 sum of t's weights over
// its routes to e, added in ascending slot order starting from 0.
__device__ __forceinline__ float token_expert_weight(const int32_t* __restrict__ ids, const float* __restrict__ tw,
                                                     int t, int k, int e) {
  float acc = 0.0f;
  for (int j = 0; j < k; ++j)
    if (ids[t * k + j] == e) acc += tw[t * k + j];
  return acc;
}

}  // namespace moeq4
