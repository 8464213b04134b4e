/*
 * Host sanitizer driver for the CPU oracle (oracle/moe_oracle.c), built with
 * AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_host_sanitizers.py.  It calls every exported oracle function on
 * small random banks of every codec and on its invalid-argument paths, and
 * checks that the per-pair, union and single-element evaluations agree
 * (they are three orders of the same fp64 sums).  Exit status 0 = clean.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_forward_pairs_q(const uint16_t *, const int32_t *, const float *, long, long, long, long, long, int, int,
                           int, const uint32_t *, const void *, const uint16_t *, const uint32_t *, const void *,
                           const uint16_t *, const uint32_t *, const void *, const uint16_t *, double *, double *,
                           double *);
int oracle_forward_union_q(const uint16_t *, const int32_t *, const float *, long, long, long, long, long, int, int,
                           int, const uint32_t *, const void *, const uint16_t *, const uint32_t *, const void *,
                           const uint16_t *, const uint32_t *, const void *, const uint16_t *, double *);
double oracle_output_element_q(const uint16_t *, const int32_t *, const float *, long, long, long, long, long, int,
                               int, int, const uint32_t *, const void *, const uint16_t *, const uint32_t *,
                               const void *, const uint16_t *, const uint32_t *, const void *, const uint16_t *, long,
                               long);
int oracle_dequant_q(int, int, int, const uint32_t *, const void *, const uint16_t *, long, long, double *);
double oracle_e4m3_value(int);
int oracle_threads(void);
void oracle_set_threads(int);

static uint64_t rs = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {
  rs = rs * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(rs >> 33);
}
static uint16_t bf16_of(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}
static float unif(void) { return (float)(rnd() % 2001) / 1000.0f - 1.0f; }

static int fails = 0;
#define CHECK(c, ...)                          \
  do {                                         \
    if (!(c)) {                                \
      fprintf(stderr, "FAIL: " __VA_ARGS__);   \
      fprintf(stderr, "\n");                   \
      ++fails;                                 \
    }                                          \
  } while (0)

static double rel(const double *a, const double *b, long n) {
  double num = 0, den = 0;
  for (long i = 0; i < n; ++i) {
    num += (a[i] - b[i]) * (a[i] - b[i]);
    den += b[i] * b[i];
  }
  return den > 0 ? sqrt(num / den) : sqrt(num);
}

/* One codec: fmt (0 affine, 1 mxfp4, 2 nvfp4, 3 mxfp8), bits, group size. */
static void codec_case(int fmt, int bits, int gs, long L, long k, long E, long H, long I) {
  const long wpr_g = H * bits / 32, wpr_d = I * bits / 32;  /* code words per row */
  const int sbytes = fmt == 0 ? 2 : 1;                        /* scale element bytes */
  const long ng = H / gs, nd = I / gs;
  uint32_t *wg = malloc(sizeof(uint32_t) * E * I * wpr_g), *wu = malloc(sizeof(uint32_t) * E * I * wpr_g);
  uint32_t *wd = malloc(sizeof(uint32_t) * E * H * wpr_d);
  unsigned char *sg = malloc((size_t)sbytes * E * I * ng), *su = malloc((size_t)sbytes * E * I * ng);
  unsigned char *sd = malloc((size_t)sbytes * E * H * nd);
  uint16_t *bg = malloc(2 * E * I * ng), *bu = malloc(2 * E * I * ng), *bd = malloc(2 * E * H * nd);
  uint16_t *x = malloc(2 * L * H);
  int32_t *ids = malloc(4 * L * k);
  float *tw = malloc(4 * L * k);
  /* E4M3 codes with bit 6 clear never spell NaN (S.1111.111) */
  const uint32_t cm = fmt == 3 ? 0xBFBFBFBFu : 0xFFFFFFFFu;
  for (long i = 0; i < E * I * wpr_g; ++i) { wg[i] = rnd() & cm; wu[i] = rnd() & cm; }
  for (long i = 0; i < E * H * wpr_d; ++i) wd[i] = rnd() & cm;
  unsigned char *sarr[3] = {sg, su, sd};
  long scount[3] = {E * I * ng, E * I * ng, E * H * nd};
  for (int a = 0; a < 3; ++a)
    for (long i = 0; i < scount[a]; ++i) {
      if (fmt == 0) {
        uint16_t v = bf16_of(0.01f + 0.02f * (float)(rnd() % 100) / 100.0f);
        memcpy(sarr[a] + 2 * i, &v, 2);
      } else if (fmt == 2) {
        sarr[a][i] = (unsigned char)(0x28 + rnd() % 0x20); /* E4M3 scales around 2^-2..2^2 */
      } else {
        sarr[a][i] = (unsigned char)(120 + rnd() % 12);    /* E8M0 2^-7..2^4 */
      }
    }
  for (long i = 0; i < E * I * ng; ++i) { bg[i] = bf16_of(-0.1f * unif()); bu[i] = bf16_of(0.1f * unif()); }
  for (long i = 0; i < E * H * nd; ++i) bd[i] = bf16_of(0.05f * unif());
  for (long i = 0; i < L * H; ++i) x[i] = bf16_of(unif());
  for (long t = 0; t < L; ++t)
    for (long j = 0; j < k; ++j) {
      ids[t * k + j] = (int32_t)(rnd() % E); /* duplicates allowed */
      tw[t * k + j] = 0.25f + (float)(rnd() % 100) / 200.0f;
    }
  const uint16_t *b_g = fmt == 0 ? bg : NULL, *b_u = fmt == 0 ? bu : NULL, *b_d = fmt == 0 ? bd : NULL;
  double *o1 = calloc(L * H, 8), *o2 = calloc(L * H, 8), *hh = calloc(L * k * I, 8), *yy = calloc(L * k * H, 8);
  int st = oracle_forward_pairs_q(x, ids, tw, L, k, E, H, I, fmt, bits, gs, wg, sg, b_g, wu, su, b_u, wd, sd, b_d,
                                  o1, hh, yy);
  CHECK(st == 0, "forward_pairs_q fmt %d bits %d gs %d status %d", fmt, bits, gs, st);
  st = oracle_forward_union_q(x, ids, tw, L, k, E, H, I, fmt, bits, gs, wg, sg, b_g, wu, su, b_u, wd, sd, b_d, o2);
  CHECK(st == 0, "forward_union_q status %d", st);
  CHECK(rel(o2, o1, L * H) <= 1e-12, "union vs pairs fmt %d: %g", fmt, rel(o2, o1, L * H));
  for (long t = 0; t < L; ++t)
    for (long m = 0; m < H; m += 37) {
      const double v = oracle_output_element_q(x, ids, tw, L, k, E, H, I, fmt, bits, gs, wg, sg, b_g, wu, su, b_u,
                                               wd, sd, b_d, t, m);
      CHECK(fabs(v - o1[t * H + m]) <= 1e-12 * (1.0 + fabs(o1[t * H + m])), "element (%ld, %ld) fmt %d", t, m, fmt);
    }
  double *dq = malloc(sizeof(double) * E * I * H);
  st = oracle_dequant_q(fmt, bits, gs, wg, sg, b_g, E * I, H, dq);
  CHECK(st == 0, "dequant_q status %d", st);
  /* invalid arguments: every call returns an error without touching memory */
  int32_t bad_ids[2] = {0, (int32_t)E};
  CHECK(oracle_forward_pairs_q(x, bad_ids, tw, 1, 2, E, H, I, fmt, bits, gs, wg, sg, b_g, wu, su, b_u, wd, sd, b_d,
                               o1, NULL, NULL) != 0, "invalid id accepted");
  CHECK(oracle_forward_pairs_q(x, ids, tw, L, k, E, H + 1, I, fmt, bits, gs, wg, sg, b_g, wu, su, b_u, wd, sd, b_d,
                               o1, NULL, NULL) != 0, "ragged H accepted");
  CHECK(oracle_forward_pairs_q(NULL, ids, tw, L, k, E, H, I, fmt, bits, gs, wg, sg, b_g, wu, su, b_u, wd, sd, b_d,
                               o1, NULL, NULL) != 0, "NULL x accepted");
  CHECK(oracle_forward_pairs_q(x, ids, tw, L, k, E, H, I, fmt, bits, 48, wg, sg, b_g, wu, su, b_u, wd, sd, b_d, o1,
                               NULL, NULL) != 0, "group 48 accepted");
  CHECK(oracle_dequant_q(fmt, bits, gs, wg, sg, b_g, 1, H + 1, dq) != 0, "dequant ragged K accepted");
  CHECK(oracle_forward_pairs_q(x, ids, tw, 0, k, E, H, I, fmt, bits, gs, wg, sg, b_g, wu, su, b_u, wd, sd, b_d, o1,
                               NULL, NULL) == 0, "L = 0 refused");
  free(wg); free(wu); free(wd); free(sg); free(su); free(sd); free(bg); free(bu); free(bd);
  free(x); free(ids); free(tw); free(o1); free(o2); free(hh); free(yy); free(dq);
}

int main(void) {
  oracle_set_threads(2);
  CHECK(oracle_threads() == 2, "threads");
  for (int b = 0; b < 256; ++b) {
    const double v = oracle_e4m3_value(b);
    CHECK(b == 0x7F || b == 0xFF ? isnan(v) : isfinite(v), "e4m3 %d", b);
  }
  codec_case(0, 4, 64, 3, 2, 4, 128, 64);
  codec_case(0, 4, 32, 2, 3, 5, 96, 160);
  codec_case(0, 8, 64, 3, 2, 4, 128, 64);
  codec_case(0, 8, 32, 2, 2, 3, 64, 96);
  codec_case(1, 4, 32, 3, 2, 4, 96, 64);
  codec_case(2, 4, 16, 2, 2, 4, 64, 96);
  codec_case(3, 8, 32, 3, 2, 4, 64, 64);
  if (fails) {
    fprintf(stderr, "%d check(s) failed\n", fails);
    return 1;
  }
  printf("oracle sanitizer driver: all checks passed\n");
  return 0;
}
