/*
 * moe_q4.h -- C ABI of the MI355X (gfx950) union-of-experts SwitchGLU library
 * over 4-bit affine, group-64 expert weights.
 *
 * One MoE layer: L tokens, each routed to k of E experts.  For every (token,
 * expert) route the layer computes the SwitchGLU of that expert -- up and gate
 * projections of x, h = silu(gate) * up, down projection of h -- and the
 * tokens' outputs are the router-weighted sums over their k routes.  Sources
 * (web pages): the SwitchGLU order and the 4-bit affine, group-64 storage come
 * from the mlx issue "gather_qmm at M=1 streams 4-bit expert weights at ~half
 * the bandwidth of M=4" (section "Numbers" and its moe_bench script); streaming
 * each distinct routed expert once for all tokens routed to it comes from the
 * mlx discussion "Small-L fused expert gather for fine-grained MoE decode"
 * (implication 1 of the section on adjacent-token overlap); the sorted
 * grouped path for large token counts and its expert-offset tile schedule come
 * from the page "MoE GatherQMM small-M verify cost" (Facts: the dispatch
 * bullets and PR 4567).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor arguments are DEVICE pointers to contiguous row-major arrays
 *   on the current HIP device.  The caller owns every buffer, including the
 *   workspace; the library never allocates, frees or synchronises in the
 *   forward calls, and enqueues all work on `stream` (NULL = default stream).
 * - Weight storage: element c of an output row is nibble c % 8 of 32-bit word
 *   c / 8, lowest nibble first; the value is scale * q + bias with q in 0..15
 *   and one bf16 (scale, bias) pair per 64 consecutive inputs of the row.
 * - Status codes are plain ints (MOE_Q4_*); nothing throws or aborts across
 *   the ABI.  Argument errors are detected on the host before any GPU work.
 * - Expert ids outside [0, E) are a precondition violation: such routes add
 *   nothing, and the kernels set MOE_Q4_DEV_BAD_ID in the workspace's device
 *   status word, which every forward call (its gate/up stage) rewrites with
 *   that call's status (see moe_q4_read_device_status).
 */
#ifndef MOE_Q4_H
#define MOE_Q4_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define MOE_Q4_OK 0
#define MOE_Q4_ERR_NULL 1        /* a required pointer is NULL                              */
#define MOE_Q4_ERR_SHAPE 2       /* L < 0, k < 1, E < 1, k > E, H or I < 1                    */
#define MOE_Q4_ERR_UNSUPPORTED 3 /* H or I not a multiple of 64, bits != 4, group != 64,      */
                                 /* out_dtype unknown, or L / E / L*k beyond the limits below */
#define MOE_Q4_ERR_ALIGN 4       /* a pointer misses its alignment (see moe_swiglu_q4_forward) */
#define MOE_Q4_ERR_WORKSPACE 5   /* workspace NULL or smaller than moe_swiglu_q4_workspace_bytes */
#define MOE_Q4_ERR_LAUNCH 6      /* a HIP launch or runtime call failed                       */
#define MOE_Q4_ERR_ALIAS 7       /* `out` overlaps an input or the workspace                  */
#define MOE_Q4_ERR_SCRATCH 8     /* the shape needs more workspace than the allocation-free   */
                                 /* entry point's scratch holds (MOE_Q4_NOALLOC_SCRATCH_BYTES) */

/* ---- device status bits (status word in the workspace header) ---- */
#define MOE_Q4_DEV_BAD_ID 1u     /* an expert id outside [0, E) was seen; its routes were dropped */

/* ---- output dtypes ---- */
#define MOE_Q4_OUT_BF16 0        /* out is bf16 [L, H], fp32 results rounded to nearest even  */
#define MOE_Q4_OUT_F32 1         /* out is fp32 [L, H] (the values before the bf16 rounding)   */

/* ---- paths (moe_swiglu_q4_select_path) ---- */
#define MOE_Q4_PATH_NONE 0       /* L == 0: nothing to do                                      */
#define MOE_Q4_PATH_UNION 1      /* small L: distinct experts streamed once, dequant GEMV       */
#define MOE_Q4_PATH_SORTED 2     /* large L: expert-sorted pairs, grouped bf16 MFMA GEMM        */

/* ---- limits ---- */
#define MOE_Q4_UNION_MAX_L 32    /* token masks are 32-bit                                     */
#define MOE_Q4_MAX_PAIRS 1024    /* L * k on the union path                                    */
#define MOE_Q4_MAX_E 16384
#define MOE_Q4_CODEC_MAX_L 65535 /* tokens of one moe_swiglu_codec_forward call          */
#define MOE_Q4_NOALLOC_SCRATCH_BYTES (16u << 20) /* scratch of moe_swiglu_q4_forward_noalloc, per GPU */

/* ---- weight codecs (moe_swiglu_codec_forward) ---- */
#define MOE_Q4_CODEC_AFFINE4_G64 0 /* 4-bit affine, bf16 scale + bias per 64 inputs (= moe_swiglu_q4_forward) */
#define MOE_Q4_CODEC_AFFINE4_G32 1 /* 4-bit affine, bf16 scale + bias per 32 inputs                      */
#define MOE_Q4_CODEC_MXFP4 2       /* FP4 E2M1 elements, one E8M0 scale byte per 32 inputs             */
#define MOE_Q4_CODEC_NVFP4 3       /* FP4 E2M1 elements, one FP8 E4M3 scale byte per 16 inputs         */
#define MOE_Q4_CODEC_AFFINE8_G64 4 /* 8-bit affine, bf16 scale + bias per 64 inputs                      */
#define MOE_Q4_CODEC_MXFP8 5       /* FP8 E4M3 elements, one E8M0 scale byte per 32 inputs             */

/* ---- forward stages (moe_swiglu_q4_forward_stages) ---- */
#define MOE_Q4_STAGE_GATEUP 1u   /* union (or sort) + fused gate/up + silu(gate)*up -> workspace  */
#define MOE_Q4_STAGE_DOWN 2u     /* down projection + router-weighted combine -> out              */
#define MOE_Q4_STAGE_ALL 3u

/*
 * Bytes of caller-provided device workspace that moe_swiglu_q4_forward needs
 * for this shape (0 for L == 0).  Returns 0 and nothing else for invalid
 * shapes as well; validate with moe_swiglu_q4_select_path.
 */
size_t moe_swiglu_q4_workspace_bytes(int L, int k, int E, int H, int I);

/*
 * Path the forward call takes for this shape (MOE_Q4_PATH_*), or a negative
 * status (-MOE_Q4_ERR_*) if the shape is invalid or unsupported.  Host only.
 * The union path serves L <= MOE_Q4_UNION_MAX_L with L * k <= MOE_Q4_MAX_PAIRS
 * (and its LDS limits); every other valid shape with L <= 65535,
 * E <= MOE_Q4_MAX_E and L * k < 2^30 takes the sorted path.
 */
int moe_swiglu_q4_select_path(int L, int k, int E, int H, int I);

/*
 * One SwitchGLU MoE layer.
 *
 *   x            bf16  [L, H]            activations                  (16-byte aligned)
 *   topk_ids     int32 [L, k]            expert of each route          (4-byte aligned)
 *   topk_weights fp32  [L, k]            router weight of each route   (4-byte aligned)
 *   wg, wu       uint32 [E, I, H/8]      gate / up codes               (16-byte aligned)
 *   sg, bg, su, bu bf16 [E, I, H/64]     gate / up scale and bias      (4-byte aligned)
 *   wd           uint32 [E, H, I/8]      down codes                    (16-byte aligned)
 *   sd, bd       bf16  [E, H, I/64]      down scale and bias           (4-byte aligned)
 *   L, k, E, H, I  tokens, routes per token, experts, hidden size, expert
 *                intermediate size; H and I multiples of 64
 *   group_size   must be 64;  bits  must be 4
 *   out          [L, H], bf16 or fp32 per out_dtype (16-byte aligned); fully
 *                overwritten, never accumulated into; must not overlap any
 *                input or the workspace
 *   workspace    device scratch of at least moe_swiglu_q4_workspace_bytes
 *                bytes (256-byte aligned); contents need no initialisation;
 *                one workspace must not serve two calls that may run at the
 *                same time
 *
 * out[t, :] = sum_j topk_weights[t, j] * Wd[e] (silu(Wg[e] x_t) * (Wu[e] x_t)),
 * e = topk_ids[t, j].  Accumulation is fp32.  The hidden vector h is never
 * rounded to bf16: the union path keeps it in fp32 and feeds the down
 * products an fp16 copy after an exact power-of-two rescale; the sorted path
 * carries it as a bf16 hi + lo pair (16 significant bits).  Results are
 * deterministic (no floating-point atomics).  L == 0 returns MOE_Q4_OK
 * without touching the GPU.
 */
int moe_swiglu_q4_forward(const void *x, const int32_t *topk_ids, const float *topk_weights,
                          const uint32_t *wg, const void *sg, const void *bg,
                          const uint32_t *wu, const void *su, const void *bu,
                          const uint32_t *wd, const void *sd, const void *bd,
                          int L, int k, int E, int H, int I, int group_size, int bits,
                          void *out, int out_dtype, void *workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * For callers that cannot allocate device memory (work recorded under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * moe_swiglu_q4_forward without the workspace arguments.  The workspace is a
 * static device array of the library, MOE_Q4_NOALLOC_SCRATCH_BYTES (16 MiB)
 * per GPU, held from the library's load until the process ends; the call
 * allocates and frees nothing.  The first call on a device looks that
 * device's copy up (hipGetSymbolAddress, with the device current).
 *
 * Arguments, results and status codes are those of moe_swiglu_q4_forward,
 * plus MOE_Q4_ERR_SCRATCH (host check, nothing enqueued) when the shape's
 * moe_swiglu_q4_workspace_bytes exceeds the scratch: every union-path shape
 * with L * k * (H + I) * 4 bytes of hidden and per-route output rows under
 * about 16 MiB fits (e.g. L = 32, k = 8, H = 6144, I = 2048), long sorted-path
 * inputs do not.
 *
 * Every call on one GPU shares that GPU's scratch, and the scratch keeps the
 * last call's contents: two calls that may run at the same time on one GPU
 * (different streams, or host threads) race and give undefined results.
 * Calls in one stream order are safe.
 */
int moe_swiglu_q4_forward_noalloc(const void *x, const int32_t *topk_ids, const float *topk_weights,
                                  const uint32_t *wg, const void *sg, const void *bg,
                                  const uint32_t *wu, const void *su, const void *bu,
                                  const uint32_t *wd, const void *sd, const void *bd,
                                  int L, int k, int E, int H, int I, int group_size, int bits,
                                  void *out, int out_dtype, hipStream_t stream);

/*
 * Same as moe_swiglu_q4_forward, restricted to the stages in `stages`
 * (MOE_Q4_STAGE_* bits).  MOE_Q4_STAGE_DOWN alone reads the hidden vectors a
 * previous MOE_Q4_STAGE_GATEUP call with identical arguments left in the same
 * workspace on the same stream.  Lets a caller time or overlap the two stages.
 */
int moe_swiglu_q4_forward_stages(const void *x, const int32_t *topk_ids, const float *topk_weights,
                                 const uint32_t *wg, const void *sg, const void *bg,
                                 const uint32_t *wu, const void *su, const void *bu,
                                 const uint32_t *wd, const void *sd, const void *bd,
                                 int L, int k, int E, int H, int I, int group_size, int bits,
                                 void *out, int out_dtype, void *workspace, size_t workspace_bytes,
                                 unsigned stages, hipStream_t stream);

/*
 * Workspace bytes moe_swiglu_codec_forward needs for this codec and shape; 0
 * if the shape is invalid or not served (see below).  Host only.
 */
size_t moe_swiglu_codec_workspace_bytes(int codec, int L, int k, int E, int H, int I);

/*
 * The same SwitchGLU MoE layer over expert banks in another weight codec
 * (MOE_Q4_CODEC_*).  The pages name these storage modes without their bit
 * layouts: mxfp4 gs32 is the format of the GLM-5.2 banks on the mlx
 * discussion page "Small-L fused expert gather for fine-grained MoE decode"
 * (section "The data", about 20 MB per expert), whose dequant-mode comparison
 * also times affine group 32; nvfp4 is among the quantized modes of PR 4572
 * on the page "MoE GatherQMM small-M verify cost" (Facts).  Layouts taken:
 *
 *   codes         4-bit codecs: element c of a row is nibble c % 8 of word
 *                 c / 8, lowest nibble first (as for moe_swiglu_q4_forward);
 *                 8-bit codecs: byte c % 4 of word c / 4, lowest byte first
 *   AFFINE4_G32   w = s * q + b, q in 0..15, bf16 s and b per 32 inputs
 *   AFFINE8_G64   w = s * q + b, q in 0..255, bf16 s and b per 64 inputs
 *   MXFP8         w = e4m3(q) * 2^(e - 127), one E8M0 byte e per 32 inputs
 *   MXFP4         w = e2m1(q) * 2^(e - 127), one E8M0 byte e per 32 inputs;
 *                 e = 255 stands for NaN (every product with that block is NaN)
 *   NVFP4         w = e2m1(q) * e4m3(s), one FP8 E4M3 byte s per 16 inputs, no
 *                 second-level scale
 *   E2M1 and E4M3 follow the OCP specifications (MX v1.0; 8-bit floating point
 *   E4M3: exponent bias 7, subnormals, S.1111.111 NaN, no infinities).
 *
 *   wg, wu      uint32 [E, I, H*bits/32]  codes                      (16-byte aligned)
 *   sg, su      [E, I, H/gs]              scales: bf16 (AFFINE4_G32, AFFINE8_G64;
 *                                         2-byte aligned), uint8 E8M0 (MXFP4, MXFP8;
 *                                         any alignment), uint8 E4M3 (NVFP4, gs = 16,
 *                                         2-byte aligned)
 *   bg, bu      bf16 [E, I, H/gs]         biases (affine codecs only, 2-byte aligned;
 *                                         ignored and may be NULL otherwise)
 *   wd, sd, bd  the same for down, [E, H, I*bits/32] and [E, H, I/gs]
 *   H, I        multiples of 32 (of 64 for AFFINE8_G64); the kernels' row steps
 *               add limits for very small H or I (a shape they cannot tile gives
 *               MOE_Q4_ERR_UNSUPPORTED and moe_swiglu_codec_workspace_bytes 0)
 *
 * All other arguments, the results' definition and the status codes are as
 * for moe_swiglu_q4_forward.  MOE_Q4_CODEC_AFFINE4_G64 is exactly
 * moe_swiglu_q4_forward (both paths).  The other codecs run on the union
 * kernels, in chunks of at most min(MOE_Q4_UNION_MAX_L, MOE_Q4_MAX_PAIRS / k)
 * tokens, fewer where that many tokens' activations do not fit one
 * workgroup's LDS (large H).  Calls with more tokens than one chunk run the
 * chunks one after another on the same workspace (sized by
 * moe_swiglu_codec_workspace_bytes); each chunk streams the distinct experts
 * of its own tokens, so long inputs re-read the bank once per chunk.  Such
 * calls need stages == MOE_Q4_STAGE_ALL.  The device status word is the OR
 * over the chunks.
 *
 * MXFP4 and MXFP8 with L > min(MOE_Q4_UNION_MAX_L, MOE_Q4_MAX_PAIRS / k) and
 * H and I multiples of 256 take the sorted path instead (expert-sorted pairs,
 * grouped bf16 MFMA GEMMs, every bank byte read once per tile row block; the
 * device path word reads MOE_Q4_PATH_SORTED; stage-split calls allowed).
 * There the scale arrays sg, su and sd must be 8-byte aligned: unaligned
 * ones run as token chunks where the shape allows that, else give
 * MOE_Q4_ERR_ALIGN.  Results are as on the union path (NaN for e = 255,
 * subnormal block scales honoured).
 *
 * L <= MOE_Q4_CODEC_MAX_L.  An unknown codec gives MOE_Q4_ERR_UNSUPPORTED.
 */
int moe_swiglu_codec_forward(int codec, const void *x, const int32_t *topk_ids, const float *topk_weights,
                             const uint32_t *wg, const void *sg, const void *bg,
                             const uint32_t *wu, const void *su, const void *bu,
                             const uint32_t *wd, const void *sd, const void *bd,
                             int L, int k, int E, int H, int I, void *out, int out_dtype,
                             void *workspace, size_t workspace_bytes, hipStream_t stream);

/* moe_swiglu_codec_forward restricted to `stages`, as moe_swiglu_q4_forward_stages. */
int moe_swiglu_codec_forward_stages(int codec, const void *x, const int32_t *topk_ids,
                                    const float *topk_weights, const uint32_t *wg, const void *sg,
                                    const void *bg, const uint32_t *wu, const void *su, const void *bu,
                                    const uint32_t *wd, const void *sd, const void *bd, int L, int k,
                                    int E, int H, int I, void *out, int out_dtype, void *workspace,
                                    size_t workspace_bytes, unsigned stages, hipStream_t stream);

/*
 * mxfp4 shorthands: moe_swiglu_codec_* with MOE_Q4_CODEC_MXFP4 and no bias
 * arrays (sg, su, sd uint8 E8M0 [.., K/32]).
 */
size_t moe_swiglu_mxfp4_workspace_bytes(int L, int k, int E, int H, int I);
int moe_swiglu_mxfp4_forward(const void *x, const int32_t *topk_ids, const float *topk_weights,
                             const uint32_t *wg, const uint8_t *sg, const uint32_t *wu, const uint8_t *su,
                             const uint32_t *wd, const uint8_t *sd, int L, int k, int E, int H, int I,
                             void *out, int out_dtype, void *workspace, size_t workspace_bytes,
                             hipStream_t stream);
int moe_swiglu_mxfp4_forward_stages(const void *x, const int32_t *topk_ids, const float *topk_weights,
                                    const uint32_t *wg, const uint8_t *sg, const uint32_t *wu,
                                    const uint8_t *su, const uint32_t *wd, const uint8_t *sd, int L, int k,
                                    int E, int H, int I, void *out, int out_dtype, void *workspace,
                                    size_t workspace_bytes, unsigned stages, hipStream_t stream);

/*
 * Union of the L * k routes (the dedup step of the union path), as its own
 * call so it can be checked bit for bit.  Outputs (device, u_max = min(E, L*k)):
 *   u            int32 [1]           number of distinct valid expert ids
 *   uniq_ids     int32 [u_max]       distinct ids ascending; -1 past u
 *   tok_mask     uint32 [u_max]      bit t set iff token t routes to uniq_ids[i]; 0 past u
 *   uniq_w       fp32 [u_max, L]     sum of token t's router weights over its routes to
 *                                    uniq_ids[i], added in ascending slot order; 0 if none
 *   slot_to_uniq int32 [L, k]        index in uniq_ids of each route; -1 for an invalid id
 * Requires 1 <= L <= MOE_Q4_UNION_MAX_L, L * k <= MOE_Q4_MAX_PAIRS, E <= MOE_Q4_MAX_E.
 */
int moe_route_union(const int32_t *topk_ids, const float *topk_weights, int L, int k, int E,
                    int32_t *u, int32_t *uniq_ids, uint32_t *tok_mask, float *uniq_w,
                    int32_t *slot_to_uniq, hipStream_t stream);

/*
 * Capacity (in tiles) that moe_sort_pairs needs for `tiles` with row tiles of
 * bm rows: L*k / bm + min(E, L*k) + 1.  Negative status for invalid arguments.
 */
int moe_sort_pairs_tiles_max(int L, int k, int E, int bm);

/*
 * Expert sort of the sorted path, as its own call so it can be checked bit for
 * bit.  Pair p = t * k + j (route j of token t).  Outputs (device):
 *   offsets  int32 [E+1]          first sorted position of each expert's pairs;
 *                                 offsets[E] = number of pairs with a valid id
 *   perm     int32 [L*k]          sorted position -> pair: valid pairs ordered by
 *                                 (expert, pair), then pairs with invalid ids by pair
 *   inv      int32 [L*k]          pair -> sorted position (inverse of perm)
 *   tiles    int32 [tiles_cap][4] row tiles (expert, first position, rows, 0):
 *                                 ceil(n_e / bm) tiles per expert, cut at expert
 *                                 boundaries, ascending expert; 16-byte aligned
 *   info     uint32 [4]           [0] MOE_Q4_DEV_* status, [1] MOE_Q4_PATH_SORTED,
 *                                 [2] valid pairs, [3] number of tiles
 *   scratch  int32 [L*k]          device scratch, contents undefined afterwards
 * tiles_cap must be at least moe_sort_pairs_tiles_max(L, k, E, bm).  The tile
 * schedule is the expert-offset one of PR 4567 described on the page "MoE
 * GatherQMM small-M verify cost" (Facts); the sort is stable in the pair index.
 */
int moe_sort_pairs(const int32_t *topk_ids, int L, int k, int E, int bm, int32_t *offsets,
                   int32_t *perm, int32_t *inv, int32_t *tiles, int tiles_cap, uint32_t *info,
                   int32_t *scratch, hipStream_t stream);

/*
 * Reads the device status word (MOE_Q4_DEV_* bits) that the last forward
 * call using this workspace left in it into *status and, if last_path is not
 * NULL, the MOE_Q4_PATH_* value that call's kernels recorded.
 * Synchronises `stream` (debug / test use, not for hot loops).
 */
int moe_q4_read_device_status(const void *workspace, uint32_t *status, uint32_t *last_path,
                              hipStream_t stream);

/* Clears the device status word (enqueued on `stream`, no sync). */
int moe_q4_clear_device_status(void *workspace, hipStream_t stream);

/*
 * Measurement reference, not part of the layer: reads `bytes` bytes of the
 * device buffer `buf` (16-byte aligned) once with 16-byte nontemporal loads,
 * the analogue of the plain streaming sum() that the mlx issue "gather_qmm at
 * M=1 streams 4-bit expert weights at ~half the bandwidth of M=4" (section
 * "Numbers") times beside its layers.  `sink` (device, 4-byte aligned) receives
 * one XOR word per workgroup and must hold at least twice the device's compute
 * unit count (sink_words); MOE_Q4_ERR_WORKSPACE otherwise.  Enqueued on
 * `stream`, no synchronisation.
 */
int moe_q4_stream_read(const void *buf, size_t bytes, uint32_t *sink, size_t sink_words, hipStream_t stream);

/* Static description of a status code; never NULL. */
const char *moe_q4_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_Q4_H */
