/*
 * CPU oracle for one SwitchGLU MoE layer over 4-bit affine, group-64 expert
 * weights.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * benchmark's CPU-baseline leg use it; the product path never does.  It shares
 * no code with the GPU library.
 *
 * What it computes (sources are the web pages named below):
 *
 *  - SwitchGLU per (token, expert) pair, in the order up, gate,
 *    silu(gate) * up, down -- mlx issue "gather_qmm at M=1 streams 4-bit expert
 *    weights at ~half the bandwidth of M=4", its moe_bench script (function
 *    moe).  silu(v) = v * sigmoid(v) = v / (1 + exp(-v)).
 *  - Each (token, expert) pair is evaluated on its own, the per-pair gather
 *    semantics described on the page "MoE GatherQMM small-M verify cost"
 *    (Facts, the gather_qmv bullets).
 *  - Dequantization is affine: w = scale * q + bias with one bf16 (scale, bias)
 *    pair per 64 consecutive inputs (the issue above, "Numbers": mx.quantize
 *    with group 64, affine, bits 4).
 *  - Storage reading (not fixed by the pages): element c of an output row is
 *    nibble c % 8 of word c / 8, lowest nibble first.
 *  - mxfp4 gs32 banks (the format of the pages' GLM-5.2 banks, mlx discussion
 *    "Small-L fused expert gather for fine-grained MoE decode", "The data";
 *    about 20 MB per expert): each 4-bit element is an FP4 E2M1 number and
 *    each 32 consecutive inputs share one 8-bit power-of-two scale.  The
 *    pages do not spell out the bit layouts; these follow the OCP
 *    Microscaling Formats (MX) specification v1.0: E2M1 = sign bit 3,
 *    exponent bits 2..1 with bias 1, mantissa bit 0, exponent 0 encoding
 *    0 and +-0.5 (no infinities or NaN); the E8M0 scale byte e stands for
 *    2^(e - 127), and e = 255 for NaN.  Packing of the elements as for the
 *    affine banks.
 *  - Further codecs named by the pages (mxfp8 in the dequant-mode comparison
 *    of the mlx discussion above; nvfp4 and mxfp8 among the quantized modes of
 *    PR 4572 on the page "MoE GatherQMM small-M verify cost", Facts; 8-bit
 *    affine models in that page's correctness reports), without their bit
 *    layouts.  The layouts taken here:
 *      affine, bits 4 or 8, group 32 or 64: w = s * q + b with unsigned q and
 *        one bf16 (s, b) per group; 8-bit codes are byte c % 4 of word c / 4,
 *        lowest byte first;
 *      nvfp4: FP4 E2M1 element (packed as the 4-bit codes) times an FP8 E4M3
 *        scale per 16 consecutive inputs, no second-level scale;
 *      mxfp8: FP8 E4M3 element (packed as the 8-bit codes) times the E8M0
 *        scale 2^(e - 127) of its 32-input block (e = 255: NaN).
 *    E4M3 follows the OCP 8-bit floating point specification: sign bit 7,
 *    exponent bits 6..3 with bias 7, mantissa bits 2..0, exponent 0 encoding
 *    subnormals m/8 * 2^-6, no infinities, and S.1111.111 the only NaN.
 *  - Router-weighted combine out[t] = sum_j w[t, j] * y[t, j] (the pages'
 *    SwitchGLU returns per-pair outputs; the weighted sum is the plain MoE
 *    combine this layer adds, applied after the down projection).
 *  - Union evaluation: the union of routed experts over the L tokens, each
 *    unique expert's weights applied once to the tokens routed to it -- mlx
 *    discussion "Small-L fused expert gather for fine-grained MoE decode",
 *    implication 1 of "The data" section.
 *
 * Precision: every step in IEEE double.  bf16 inputs widen exactly; q, scale
 * and bias products are exact in double; dot products accumulate in ascending
 * index order.  No -ffast-math.
 *
 * Threading: OpenMP splits independent output elements (pairs x rows) across
 * threads; no reduction is split, so results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_EINVAL 1
#define ORC_ENOMEM 2

static double bf16_to_double(uint16_t h) {
    uint32_t bits = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* 4-bit code of input element c in a packed row. */
static unsigned code_at(const uint32_t *row_words, long c) {
    return (row_words[c / 8] >> (4 * (c % 8))) & 0xFu;
}

/* Value of a 4-bit FP4 E2M1 code (OCP MX v1.0 element encoding). */
static double e2m1_value(unsigned code) {
    unsigned sign = (code >> 3) & 1u, expo = (code >> 1) & 3u, mant = code & 1u;
    double mag = expo == 0 ? 0.5 * (double)mant : ldexp(1.0 + 0.5 * (double)mant, (int)expo - 1);
    return sign ? -mag : mag;
}

/* mxfp4 weight at (row, c): E2M1 element times the block's 2^(e - 127). */
static double weight_at_mx(const uint32_t *W, const uint8_t *S, long row, long K, long c) {
    unsigned e = S[row * (K / 32) + c / 32];
    if (e == 255u) return NAN;
    return ldexp(e2m1_value(code_at(W + row * (K / 8), c)), (int)e - 127);
}

/* 8-bit code of input element c in a packed row. */
static unsigned code8_at(const uint32_t *row_words, long c) {
    return (row_words[c / 4] >> (8 * (c % 4))) & 0xFFu;
}

/* Value of an FP8 E4M3 number (OCP 8-bit floating point, E4M3 variant). */
static double e4m3_value(unsigned b) {
    unsigned sign = (b >> 7) & 1u, expo = (b >> 3) & 15u, mant = b & 7u;
    if (expo == 15u && mant == 7u) return NAN;
    double mag = expo == 0 ? ldexp((double)mant / 8.0, -6) : ldexp(1.0 + (double)mant / 8.0, (int)expo - 7);
    return sign ? -mag : mag;
}

#define ORC_FMT_AFFINE 0
#define ORC_FMT_MXFP4 1
#define ORC_FMT_NVFP4 2
#define ORC_FMT_MXFP8 3

/* One quantized matrix of a codec: codes, per-group scales, per-group biases (affine only). */
typedef struct {
    int fmt, bits, gs;
    const uint32_t *W;
    const void *S;
    const uint16_t *B;
} qmat_t;

/* Dequantized weight at (row, c) of a matrix with K inputs per row, any codec. */
static double weight_at_q(const qmat_t *m, long row, long K, long c) {
    const uint8_t *S8 = (const uint8_t *)m->S;
    switch (m->fmt) {
    case ORC_FMT_AFFINE: {
        long g = row * (K / m->gs) + c / m->gs;
        const uint32_t *rw = m->W + row * (K * m->bits / 32);
        unsigned q = m->bits == 8 ? code8_at(rw, c) : code_at(rw, c);
        return bf16_to_double(((const uint16_t *)m->S)[g]) * (double)q + bf16_to_double(m->B[g]);
    }
    case ORC_FMT_MXFP4:
        return weight_at_mx(m->W, S8, row, K, c);
    case ORC_FMT_NVFP4:
        return e2m1_value(code_at(m->W + row * (K / 8), c)) * e4m3_value(S8[row * (K / 16) + c / 16]);
    case ORC_FMT_MXFP8: {
        unsigned e = S8[row * (K / 32) + c / 32];
        if (e == 255u) return NAN;
        return ldexp(e4m3_value(code8_at(m->W + row * (K / 4), c)), (int)e - 127);
    }
    }
    return NAN;
}

/* Inputs per scale group of a codec, or 0 if the (fmt, bits, gs) triple is not one. */
static long codec_group(int fmt, int bits, int gs) {
    switch (fmt) {
    case ORC_FMT_AFFINE: return (bits == 4 || bits == 8) && (gs == 32 || gs == 64) ? gs : 0;
    case ORC_FMT_MXFP4: return bits == 4 && gs == 32 ? 32 : 0;
    case ORC_FMT_NVFP4: return bits == 4 && gs == 16 ? 16 : 0;
    case ORC_FMT_MXFP8: return bits == 8 && gs == 32 ? 32 : 0;
    }
    return 0;
}

static double silu(double v) { return v / (1.0 + exp(-v)); }

int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* The three quantized matrices of one layer's experts: gate, up, down (one codec). */
typedef struct {
    qmat_t m[3];
} bank_t;

/* Weight of matrix mat (0 gate, 1 up, 2 down) at (row, c). */
static double bank_weight(const bank_t *bk, int mat, long row, long K, long c) {
    return weight_at_q(&bk->m[mat], row, K, c);
}

/* Hidden activation of one (token, expert) pair: h[n] = silu(gate[n]) * up[n]. */
static double pair_hidden_row(const bank_t *bk, const uint16_t *xrow, long e, long H, long I, long n) {
    long row = e * I + n;
    double g = 0.0, u = 0.0;
    for (long c = 0; c < H; ++c) {
        double xc = bf16_to_double(xrow[c]);
        u += xc * bank_weight(bk, 1, row, H, c);
        g += xc * bank_weight(bk, 0, row, H, c);
    }
    return silu(g) * u;
}

/* Down projection of one pair's hidden vector: y[m] = sum_n h[n] * Wd[e, m, n]. */
static double pair_down_row(const bank_t *bk, const double *h, long e, long H, long I, long m) {
    long row = e * H + m;
    double y = 0.0;
    for (long n = 0; n < I; ++n) y += h[n] * bank_weight(bk, 2, row, I, n);
    return y;
}

static int check_shapes_q(const int32_t *ids, long L, long k, long E, long H, long I, long q) {
    if (L < 0 || k <= 0 || E <= 0 || H <= 0 || I <= 0 || H % q || I % q) return ORC_EINVAL;
    for (long p = 0; p < L * k; ++p)
        if (ids[p] < 0 || ids[p] >= E) return ORC_EINVAL;
    return ORC_OK;
}

/*
 * Per-pair evaluation.  x bf16 [L, H]; ids int32 [L, k]; tw fp32 [L, k];
 * the bank's matrices gate/up [E, I, .] and down [E, H, .].  Writes out[L, H]
 * (double).  If h_out is not NULL it also gets
 * every pair's hidden vector, h_out[(t * k + j) * I + n]; if y_out is not NULL,
 * every pair's down output y_out[(t * k + j) * H + m].
 */
static int forward_pairs_bank(const uint16_t *x, const int32_t *ids, const float *tw,
                              long L, long k, long H, long I, const bank_t *bkp,
                              double *out, double *h_out, double *y_out) {
    const bank_t bk = *bkp;
    long P = L * k;
    double *h = (double *)malloc(sizeof(double) * (size_t)(P > 0 ? P : 1) * (size_t)I);
    double *y = (double *)malloc(sizeof(double) * (size_t)(P > 0 ? P : 1) * (size_t)H);
    if (!h || !y) { free(h); free(y); return ORC_ENOMEM; }

    /* gate, up, silu(gate) * up for every pair and hidden row */
#pragma omp parallel for schedule(dynamic, 16)
    for (long pn = 0; pn < P * I; ++pn) {
        long p = pn / I, n = pn % I;
        h[pn] = pair_hidden_row(&bk, x + (p / k) * H, ids[p], H, I, n);
    }
    /* down projection for every pair and output row */
#pragma omp parallel for schedule(dynamic, 16)
    for (long pm = 0; pm < P * H; ++pm) {
        long p = pm / H, m = pm % H;
        y[pm] = pair_down_row(&bk, h + p * I, ids[p], H, I, m);
    }
    /* router-weighted combine, ascending slot order */
    for (long t = 0; t < L; ++t)
        for (long m = 0; m < H; ++m) {
            double acc = 0.0;
            for (long j = 0; j < k; ++j) acc += (double)tw[t * k + j] * y[(t * k + j) * H + m];
            out[t * H + m] = acc;
        }
    if (h_out) memcpy(h_out, h, sizeof(double) * (size_t)P * (size_t)I);
    if (y_out) memcpy(y_out, y, sizeof(double) * (size_t)P * (size_t)H);
    free(h);
    free(y);
    return ORC_OK;
}

/*
 * Union evaluation: the distinct experts of all L * k routes, ascending; each
 * one's hidden and down vectors computed once per token routed to it, then
 * added with that token's summed router weight for the expert.  Same
 * arguments and output as forward_pairs_bank.
 */
static int forward_union_bank(const uint16_t *x, const int32_t *ids, const float *tw,
                              long L, long k, long H, long I, const bank_t *bkp, double *out) {
    const bank_t bk = *bkp;
    long P = L * k;

    /* distinct expert ids, ascending (insertion into a sorted list) */
    long *uniq = (long *)malloc(sizeof(long) * (size_t)(P > 0 ? P : 1));
    long u = 0;
    for (long p = 0; p < P; ++p) {
        long e = ids[p], pos = 0;
        while (pos < u && uniq[pos] < e) ++pos;
        if (pos < u && uniq[pos] == e) continue;
        for (long q = u; q > pos; --q) uniq[q] = uniq[q - 1];
        uniq[pos] = e;
        ++u;
    }
    /* (unique expert, token) pairs that carry weight, with that weight */
    long *pe = (long *)malloc(sizeof(long) * (size_t)(P > 0 ? P : 1));
    long *pt = (long *)malloc(sizeof(long) * (size_t)(P > 0 ? P : 1));
    double *pw = (double *)malloc(sizeof(double) * (size_t)(P > 0 ? P : 1));
    long np = 0;
    for (long i = 0; i < u; ++i)
        for (long t = 0; t < L; ++t) {
            double wsum = 0.0;
            int hit = 0;
            for (long j = 0; j < k; ++j)
                if (ids[t * k + j] == uniq[i]) { wsum += (double)tw[t * k + j]; hit = 1; }
            if (hit) { pe[np] = uniq[i]; pt[np] = t; pw[np] = wsum; ++np; }
        }
    double *h = (double *)malloc(sizeof(double) * (size_t)(np > 0 ? np : 1) * (size_t)I);
    double *y = (double *)malloc(sizeof(double) * (size_t)(np > 0 ? np : 1) * (size_t)H);
    if (!uniq || !pe || !pt || !pw || !h || !y) {
        free(uniq); free(pe); free(pt); free(pw); free(h); free(y);
        return ORC_ENOMEM;
    }
#pragma omp parallel for schedule(dynamic, 16)
    for (long qn = 0; qn < np * I; ++qn) {
        long q = qn / I, n = qn % I;
        h[qn] = pair_hidden_row(&bk, x + pt[q] * H, pe[q], H, I, n);
    }
#pragma omp parallel for schedule(dynamic, 16)
    for (long qm = 0; qm < np * H; ++qm) {
        long q = qm / H, m = qm % H;
        y[qm] = pair_down_row(&bk, h + q * I, pe[q], H, I, m);
    }
    for (long i = 0; i < L * H; ++i) out[i] = 0.0;
    for (long q = 0; q < np; ++q)
        for (long m = 0; m < H; ++m) out[pt[q] * H + m] += pw[q] * y[q * H + m];
    free(uniq); free(pe); free(pt); free(pw); free(h); free(y);
    return ORC_OK;
}

/*
 * One output element computed on its own: out[t, m] for token t and output
 * row m, per-pair evaluation.  Lets tests sample single outputs of full-size
 * layers.
 */
static double output_element_bank(const uint16_t *x, const int32_t *ids, const float *tw, long k, long H, long I,
                                  const bank_t *bk, long t, long m) {
    double *h = (double *)malloc(sizeof(double) * (size_t)I);
    if (!h) return NAN;
    double acc = 0.0;
    for (long j = 0; j < k; ++j) {
        long e = ids[t * k + j];
#pragma omp parallel for schedule(static)
        for (long n = 0; n < I; ++n) h[n] = pair_hidden_row(bk, x + t * H, e, H, I, n);
        acc += (double)tw[t * k + j] * pair_down_row(bk, h, e, H, I, m);
    }
    free(h);
    return acc;
}

/*
 * The entry points, for any codec (ORC_FMT_* with its bits and group size; the
 * 4-bit affine group-64 banks are ORC_FMT_AFFINE, 4, 64): the per-pair, union
 * and single-element evaluations and a dense dequantized copy.  The
 * single-element form returns NAN on invalid arguments.  Codes are packed
 * uint32 words [rows, K * bits / 32]; scales are bf16 (affine) or uint8 (the
 * others) [rows, K / gs]; biases bf16 [rows, K / gs] for affine, else unused.
 */
static int make_bank_q(bank_t *bk, int fmt, int bits, int gs,
                       const uint32_t *wg, const void *sg, const uint16_t *bg,
                       const uint32_t *wu, const void *su, const uint16_t *bu,
                       const uint32_t *wd, const void *sd, const uint16_t *bd) {
    if (!codec_group(fmt, bits, gs)) return ORC_EINVAL;
    if (!wg || !sg || !wu || !su || !wd || !sd) return ORC_EINVAL;
    if (fmt == ORC_FMT_AFFINE && (!bg || !bu || !bd)) return ORC_EINVAL;
    memset(bk, 0, sizeof *bk);
    const uint32_t *w[3] = {wg, wu, wd};
    const void *sc[3] = {sg, su, sd};
    const uint16_t *bi[3] = {bg, bu, bd};
    for (int i = 0; i < 3; ++i) {
        bk->m[i].fmt = fmt; bk->m[i].bits = bits; bk->m[i].gs = gs;
        bk->m[i].W = w[i]; bk->m[i].S = sc[i]; bk->m[i].B = bi[i];
    }
    return ORC_OK;
}

int oracle_forward_pairs_q(const uint16_t *x, const int32_t *ids, const float *tw,
                           long L, long k, long E, long H, long I, int fmt, int bits, int gs,
                           const uint32_t *wg, const void *sg, const uint16_t *bg,
                           const uint32_t *wu, const void *su, const uint16_t *bu,
                           const uint32_t *wd, const void *sd, const uint16_t *bd,
                           double *out, double *h_out, double *y_out) {
    bank_t bk;
    if (!out || (L > 0 && (!x || !ids || !tw))) return ORC_EINVAL;
    if (make_bank_q(&bk, fmt, bits, gs, wg, sg, bg, wu, su, bu, wd, sd, bd)) return ORC_EINVAL;
    int st = check_shapes_q(ids, L, k, E, H, I, codec_group(fmt, bits, gs));
    if (st) return st;
    return forward_pairs_bank(x, ids, tw, L, k, H, I, &bk, out, h_out, y_out);
}

int oracle_forward_union_q(const uint16_t *x, const int32_t *ids, const float *tw,
                           long L, long k, long E, long H, long I, int fmt, int bits, int gs,
                           const uint32_t *wg, const void *sg, const uint16_t *bg,
                           const uint32_t *wu, const void *su, const uint16_t *bu,
                           const uint32_t *wd, const void *sd, const uint16_t *bd, double *out) {
    bank_t bk;
    if (!out || (L > 0 && (!x || !ids || !tw))) return ORC_EINVAL;
    if (make_bank_q(&bk, fmt, bits, gs, wg, sg, bg, wu, su, bu, wd, sd, bd)) return ORC_EINVAL;
    int st = check_shapes_q(ids, L, k, E, H, I, codec_group(fmt, bits, gs));
    if (st) return st;
    return forward_union_bank(x, ids, tw, L, k, H, I, &bk, out);
}

double oracle_output_element_q(const uint16_t *x, const int32_t *ids, const float *tw,
                               long L, long k, long E, long H, long I, int fmt, int bits, int gs,
                               const uint32_t *wg, const void *sg, const uint16_t *bg,
                               const uint32_t *wu, const void *su, const uint16_t *bu,
                               const uint32_t *wd, const void *sd, const uint16_t *bd, long t, long m) {
    bank_t bk;
    if (make_bank_q(&bk, fmt, bits, gs, wg, sg, bg, wu, su, bu, wd, sd, bd)) return NAN;
    if (t < 0 || t >= L || m < 0 || m >= H || check_shapes_q(ids, L, k, E, H, I, codec_group(fmt, bits, gs)))
        return NAN;
    return output_element_bank(x, ids, tw, k, H, I, &bk, t, m);
}

int oracle_dequant_q(int fmt, int bits, int gs, const uint32_t *W, const void *S, const uint16_t *B,
                     long rows, long K, double *out) {
    long g = codec_group(fmt, bits, gs);
    if (!g || !W || !S || !out || (fmt == ORC_FMT_AFFINE && !B) || rows < 0 || K <= 0 || K % g) return ORC_EINVAL;
    qmat_t m = {fmt, bits, gs, W, S, B};
    for (long r = 0; r < rows; ++r)
        for (long c = 0; c < K; ++c) out[r * K + c] = weight_at_q(&m, r, K, c);
    return ORC_OK;
}

/* Value of one E4M3 byte (exported for the pins of the codec tables). */
double oracle_e4m3_value(int b) { return e4m3_value((unsigned)b & 0xFFu); }
