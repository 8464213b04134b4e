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

// Four copies of the high byte of bf16 128.0 (0x4300).  A byte permute that
// places a 4-bit code q under each copy yields the bf16 value 128 + q exactly
// (bf16 has 7 mantissa bits; at exponent 2^7 one mantissa step is 1).
constexpr uint32_t kMagicBytes = 0x43434343u;
// Same for fp16 1024.0 (0x6400): 10 mantissa bits, one step is 1 at 2^10.
constexpr uint32_t kMagicBytesF16 = 0x64646464u;

// Splits one 32-bit word of eight codes (nibble c holds element c) into four
// bf16 pairs (low half, high half):
//   out[0] = (128+q0, 128+q2)  out[1] = (128+q4, 128+q6)
//   out[2] = (128+q1, 128+q3)  out[3] = (128+q5, 128+q7)
// Three mask/shift ops isolate the even and odd nibbles as bytes; each pair
// is then one v_perm_b32 that interleaves two of those bytes with 0x43 bytes.
__device__ __forceinline__ void unpack_word(uint32_t w, uint32_t magic, uint32_t out[4]) {
  const uint32_t ev = w & 0x0F0F0F0Fu;          // bytes: q0 q2 q4 q6
  const uint32_t od = (w >> 4) & 0x0F0F0F0Fu;   // bytes: q1 q3 q5 q7
  // selector bytes 0-3 pick bytes of the second operand, 4-7 of the first
  out[0] = __builtin_amdgcn_perm(magic, ev, 0x04010400u);
  out[1] = __builtin_amdgcn_perm(magic, ev, 0x04030402u);
  out[2] = __builtin_amdgcn_perm(magic, od, 0x04010400u);
  out[3] = __builtin_amdgcn_perm(magic, od, 0x04030402u);
}

// acc + a.lo * b.lo + a.hi * b.hi with bf16 inputs and fp32 accumulation
// (v_dot2c_f32_bf16; bf16 x bf16 products are exact in fp32).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b),
                                         acc, false);
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// acc + a.lo * b.lo + a.hi * b.hi with fp16 inputs and fp32 accumulation
// (v_dot2c_f32_f16; fp16 x fp16 products are exact in fp32).
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), acc, false);
}

// mxfp4 gs32 (OCP MX: FP4 E2M1 elements, one E8M0 scale byte per 32 inputs).
// gfx950 converts the two E2M1 codes of one byte (low nibble first) to a
// bf16 or fp16 pair exactly (scale operand 1.0); the block's 2^(e - 127)
// multiplies the fp32 partial sum of its 32 products afterwards.
// Sum of the 32 products of one position: codes w (8 per word, element c in
// nibble c of its word) against 16 bf16 pairs in natural element order.
__device__ __forceinline__ float dot32_mx_bf16(const uint4 w, const uint32_t (&av)[16], float d) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(ws[i], 1.0f, 0),
                                        __builtin_bit_cast(bf16x2_t, av[4 * i + 0]), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(ws[i], 1.0f, 1),
                                        __builtin_bit_cast(bf16x2_t, av[4 * i + 1]), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(ws[i], 1.0f, 2),
                                        __builtin_bit_cast(bf16x2_t, av[4 * i + 2]), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(ws[i], 1.0f, 3),
                                        __builtin_bit_cast(bf16x2_t, av[4 * i + 3]), d, false);
  }
  return d;
}

// The same against 16 fp16 pairs in natural element order.
__device__ __forceinline__ float dot32_mx_f16(const uint4 w, const uint32_t (&hv)[16], float d) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    d = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ws[i], 1.0f, 0),
                               __builtin_bit_cast(half2_t, hv[4 * i + 0]), d, false);
    d = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ws[i], 1.0f, 1),
                               __builtin_bit_cast(half2_t, hv[4 * i + 1]), d, false);
    d = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ws[i], 1.0f, 2),
                               __builtin_bit_cast(half2_t, hv[4 * i + 2]), d, false);
    d = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ws[i], 1.0f, 3),
                               __builtin_bit_cast(half2_t, hv[4 * i + 3]), d, false);
  }
  return d;
}

// A block's partial sum times its E8M0 scale 2^(e - 127); e = 255 is NaN.
// nvfp4: the same products split at the 16-input scale boundary; elements
// 0..15 sit in words 0 and 1, elements 16..31 in words 2 and 3.  Returns
// s0 * (first 16 products) + s1 * (last 16 products).
__device__ __forceinline__ float dot32_nv_bf16(const uint4 w, const uint32_t (&av)[16], float s0, float s1) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  float d[2] = {0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float& e = d[i >> 1];
    e = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(ws[i], 1.0f, 0),
                                        __builtin_bit_cast(bf16x2_t, av[4 * i + 0]), e, false);
    e = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(ws[i], 1.0f, 1),
                                        __builtin_bit_cast(bf16x2_t, av[4 * i + 1]), e, false);
    e = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(ws[i], 1.0f, 2),
                                        __builtin_bit_cast(bf16x2_t, av[4 * i + 2]), e, false);
    e = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(ws[i], 1.0f, 3),
                                        __builtin_bit_cast(bf16x2_t, av[4 * i + 3]), e, false);
  }
  return __builtin_fmaf(d[1], s1, d[0] * s0);
}

__device__ __forceinline__ float dot32_nv_f16(const uint4 w, const uint32_t (&hv)[16], float s0, float s1) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  float d[2] = {0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float& e = d[i >> 1];
    e = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ws[i], 1.0f, 0),
                               __builtin_bit_cast(half2_t, hv[4 * i + 0]), e, false);
    e = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ws[i], 1.0f, 1),
                               __builtin_bit_cast(half2_t, hv[4 * i + 1]), e, false);
    e = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ws[i], 1.0f, 2),
                               __builtin_bit_cast(half2_t, hv[4 * i + 2]), e, false);
    e = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ws[i], 1.0f, 3),
                               __builtin_bit_cast(half2_t, hv[4 * i + 3]), e, false);
  }
  return __builtin_fmaf(d[1], s1, d[0] * s0);
}

// 8-bit codes: a 16-byte load holds 16 elements (element c is byte c % 4 of
// word c / 4, lowest byte first), against 8 activation pairs in natural order.
//
// Affine 8-bit against bf16 pairs: each byte q = l + 16 h is split into its
// nibbles, each placed under the bf16 128 exponent as for 4-bit codes, so
// the sum of the 16 products comes out as sum_c a_c * (q_c + 2176) with
// 2176 = 128 * (1 + 16), exact products and fp32 accumulation.
__device__ __forceinline__ float dot16_a8_bf16(const uint4 w, const uint32_t (&av)[16], float d) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  float dl = 0.0f, dh = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t q[4];
    unpack_word(ws[i], kMagicBytes, q);  // (l0,l1), (l2,l3), (h0,h1), (h2,h3) of the word's bytes
    dl = dot2_bf16(q[0], av[2 * i], dl);
    dl = dot2_bf16(q[1], av[2 * i + 1], dl);
    dh = dot2_bf16(q[2], av[2 * i], dh);
    dh = dot2_bf16(q[3], av[2 * i + 1], dh);
  }
  return __builtin_fmaf(16.0f, dh, dl + d);
}

// Affine 8-bit against fp16 pairs: a byte under the fp16 1024 exponent is
// 1024 + q exactly, two per v_perm; sum_c h_c * (q_c + 1024).
__device__ __forceinline__ float dot16_a8_f16(const uint4 w, const uint32_t (&hv)[16], float d) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // selector bytes 0-3 pick bytes of the second operand, 4-7 of the first
    d = dot2_f16(__builtin_amdgcn_perm(kMagicBytesF16, ws[i], 0x04010400u), hv[2 * i], d);
    d = dot2_f16(__builtin_amdgcn_perm(kMagicBytesF16, ws[i], 0x04030402u), hv[2 * i + 1], d);
  }
  return d;
}

// mxfp8 (OCP MX: FP8 E4M3 elements, E8M0 scale per 32 inputs): gfx950's
// scaled FP8 conversions turn two E4M3 bytes (word_sel false: bytes 0 and 1,
// true: bytes 2 and 3) into an exact bf16 / fp16 pair (scale operand 1.0).
__device__ __forceinline__ float dot16_mx8_bf16(const uint4 w, const uint32_t (&av)[16], float d) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ws[i], 1.0f, false),
                                        __builtin_bit_cast(bf16x2_t, av[2 * i]), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ws[i], 1.0f, true),
                                        __builtin_bit_cast(bf16x2_t, av[2 * i + 1]), d, false);
  }
  return d;
}

__device__ __forceinline__ float dot16_mx8_f16(const uint4 w, const uint32_t (&hv)[16], float d) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    d = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(ws[i], 1.0f, false),
                               __builtin_bit_cast(half2_t, hv[2 * i]), d, false);
    d = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(ws[i], 1.0f, true),
                               __builtin_bit_cast(half2_t, hv[2 * i + 1]), d, false);
  }
  return d;
}

// Value of an FP8 E4M3 byte (OCP: exponent bias 7, three mantissa bits,
// exponent 0 subnormal, S.1111.111 NaN), exact in fp32: a normal number's
// fields move into the fp32 fields; a subnormal m/8 * 2^-6 is m * 2^-9.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  const float mag = e ? __builtin_bit_cast(float, ((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
  const float v = (b & 0x80u) ? -mag : mag;
  return (e == 15u && m == 7u) ? __builtin_nanf("") : v;
}

__device__ __forceinline__ float mx_scaled(float d, uint32_t e) {
  return e == 255u ? __builtin_nanf("") : __builtin_amdgcn_ldexpf(d, (int)e - 127);
}

// Value of lane 4*(lane/4) + A of the caller's quad (DPP quad_perm broadcast).
template <int A>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, A * 0x55, 0xF, 0xF, false);
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
// (e0,e2), (e4,e6), (e1,e3), (e5,e7).
__device__ __forceinline__ uint4 pair_activations(uint4 v) {
  uint4 r;
  r.x = (v.x & 0xFFFFu) | (v.y << 16);
  r.y = (v.z & 0xFFFFu) | (v.w << 16);
  r.z = (v.x >> 16) | (v.y & 0xFFFF0000u);
  r.w = (v.z >> 16) | (v.w & 0xFFFF0000u);
  return r;
}

// Element index (0..7) of the low and high halves of pair kk produced by
// unpack_word / pair_activations.
__device__ __forceinline__ constexpr int pair_lo(int kk) { return (kk & 2) ? ((kk & 1) ? 5 : 1) : ((kk & 1) ? 4 : 0); }
__device__ __forceinline__ constexpr int pair_hi(int kk) { return pair_lo(kk) + 2; }

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

// Maximum over the 64 lanes of a wave; every lane receives it.
// Totals of RS rows whose partial sums are spread over the LPR lanes of each
// lane group (v[r]: this lane's part of row r).  Reduce-scatter over the
// quad (each exchange halves the values a lane carries), then an all-reduce
// over the lanes that carry the same row.  Lane li of a group returns the
// total of row li % RS; every lane with that residue holds the same value.
template <int LPR, int RS>
__device__ __forceinline__ float reduce_rows(const float (&v)[RS]) {
  static_assert(RS == 2 || RS == 4, "rows per group");
  static_assert(LPR >= RS && LPR <= 64, "lanes per group");
  const int lane = threadIdx.x & 63;
  const bool b0 = lane & 1, b1 = lane & 2;
  float k;
  if constexpr (RS == 4) {
    float k0 = b0 ? v[1] : v[0];
    float k1 = b0 ? v[3] : v[2];
    k0 += dpp_f32<0xB1>(b0 ? v[0] : v[1]);  // quad_perm(1,0,3,2): lane ^ 1
    k1 += dpp_f32<0xB1>(b0 ? v[2] : v[3]);
    k = b1 ? k1 : k0;
    k += dpp_f32<0x4E>(b1 ? k0 : k1);      // quad_perm(2,3,0,1): lane ^ 2
  } else {
    k = b0 ? v[1] : v[0];
    k += dpp_f32<0xB1>(b0 ? v[0] : v[1]);
    if constexpr (LPR >= 4) k += dpp_f32<0x4E>(k);
  }
  if constexpr (LPR == 8) k += __shfl_xor(k, 4, 64);
  if constexpr (LPR >= 16) {
    k += dpp_f32<0x124>(k);  // row_ror:4 (the 4 quads of a 16-lane row)
    k += dpp_f32<0x128>(k);  // row_ror:8
  }
  if constexpr (LPR >= 32) {
    const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(k), __float_as_uint(k), false, false);
    k = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);  // rows 0 + 1, rows 2 + 3
  }
  if constexpr (LPR == 64) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(k), __float_as_uint(k), false, false);
    k = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);  // lanes 0-31 + lanes 32-63
  }
  return k;
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  v = fmaxf(v, dpp_f32<0x140>(v));
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  v = fmaxf(v, __shfl_xor(v, 32, 64));
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

// Index of the n-th set bit (n counted from 0) of m; m has more than n bits
// set.  Binary search by population counts of the low halves (five steps,
// no loop over the bits).
__device__ __forceinline__ int nth_set_bit(uint32_t m, int n) {
  int base = 0;
#pragma unroll
  for (int w = 16; w >= 1; w >>= 1) {
    const uint32_t lo = m & ((1u << w) - 1u);
    const int c = __popc(lo);
    const bool up = n >= c;
    n = up ? n - c : n;
    m = up ? m >> w : lo;
    base += up ? w : 0;
  }
  return base;
}

// Union of the routes, built in LDS by one workgroup.
//   bitmap[EW]  presence of each expert id      scan[EW]  exclusive popcount prefix
//   uniq[P]     distinct ids ascending          mask[P]   token mask per distinct id
//   off[P+1]    exclusive prefix of popcount(mask): first pair slot of each distinct id
//   scal[0] = u (distinct ids), scal[1] = 1 if an id fell outside [0, E)
//   ids[P], tw[P]  the routes and their router weights, staged by stage_routes
struct UnionLds {
  uint32_t* bitmap;
  int32_t* scan;
  int32_t* uniq;
  uint32_t* mask;
  int32_t* off;
  int32_t* scal;
  int32_t* ids;
  float* tw;
};

// Copies the routes into LDS (no barrier; build_union's first barrier
// publishes them).  Issued first so the loads overlap whatever follows.
__device__ __forceinline__ void stage_routes(const int32_t* __restrict__ ids, const float* __restrict__ tw, int P,
                                             const UnionLds& s) {
  for (int p = threadIdx.x; p < P; p += blockDim.x) {
    s.ids[p] = ids[p];
    s.tw[p] = tw[p];
  }
}

// Every thread of the workgroup must call this (it contains barriers), after
// stage_routes.  Requires blockDim.x >= 64, L <= 32, P = L * k.
__device__ inline void build_union(int P, int k, int E, const UnionLds& s) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int EW = (E + 31) >> 5;
  for (int w = tid; w < EW; w += nthr) s.bitmap[w] = 0u;
  for (int i = tid; i < P; i += nthr) s.mask[i] = 0u;
  if (tid == 0) s.scal[1] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += nthr) {
    const int e = s.ids[p];
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
    const int e = s.ids[p];
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
// its routes to e, added in ascending slot order starting from 0 (routes
// read from the LDS copy).
__device__ __forceinline__ float token_expert_weight(const UnionLds& s, int t, int k, int e) {
  float acc = 0.0f;
  for (int j = 0; j < k; ++j)
    if (s.ids[t * k + j] == e) acc += s.tw[t * k + j];
  return acc;
}

// Buffer resource: a wave-uniform 128-bit descriptor (base address, byte
// range) in scalar registers plus a 32-bit per-lane offset keeps address
// arithmetic off the vector ALU.  A load past the range returns zero without
// touching memory, which lets the streaming loops issue every prefetch
// unconditionally (a zero range turns it into a no-op).
typedef int v4i_t __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;
// cache-policy operand of the buffer-load builtins: bit 1 is `nt` on gfx950
constexpr int kCpolNt = 2;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // raw (unformatted) buffer, stride 0: 0x00020000 is the data-format word of
  // such a resource on gfx9-family parts
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// Expert weights are read once per launch. The nontemporal hint (`nt`) marks
// their lines for early eviction, so the weight stream does not push the
// reused activations, scale rows and hidden vectors out of the caches
// (measured: 3-4 % less layer time at every L).
__device__ __forceinline__ uint4 bld16_nt(rsrc_t r, uint32_t off) {
  const v4i_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolNt);
  return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
}
__device__ __forceinline__ uint4 ld16_nt(const unsigned char* p) {
  const v4i_t v = __builtin_nontemporal_load(reinterpret_cast<const v4i_t*>(p));
  return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
}
__device__ __forceinline__ uint32_t bld2(rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t bld1(rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}
typedef unsigned int u32x2_b_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2_b_t bld8(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2_b_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}

}  // namespace moeq4
