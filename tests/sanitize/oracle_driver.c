/* Drives every entry point of the fp64 oracle (oracle/helm_oracle.c) on tiny
 * inputs, both storage types, valid and invalid arguments, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitizers.py).
 * Test infrastructure: it checks memory and undefined-behaviour safety, not
 * values (the pins do that).  Exit status 0 = every call returned what it
 * should. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* the oracle's argument structures (oracle/helm_oracle.c) */
typedef struct {
  int32_t n_src_layers, n_tgt_layers, n_kv_heads, head_dim, k, dtype, quantize_content, n_threads;
  int64_t n_tokens;
  double theta_src, theta_tgt;
} oracle_problem;
typedef struct {
  int32_t block_size, n_requests, max_blocks_src, max_blocks_tgt, n_src_blocks, n_tgt_blocks;
} oracle_paged;

double oracle_round_bf16(double x);
int oracle_transfer_rows(const oracle_problem*, const void*, const void*, const int32_t*, const int32_t*,
                         const int32_t*, const void*, const float*, const void*, const float*, int64_t,
                         const int64_t*, double*, double*);
int oracle_transfer_wide_rows(const oracle_problem*, const void*, const void*, const int32_t*, const int32_t*,
                              const int32_t*, const void*, const float*, const void*, const float*, int64_t,
                              const int64_t*, double*, double*);
int oracle_transfer_paged_rows(const oracle_problem*, const oracle_paged*, const void*, const void*,
                               const int32_t*, const int32_t*, const int32_t*, const int32_t*, const int32_t*,
                               const int32_t*, const void*, const float*, const void*, const float*, int64_t,
                               const int64_t*, double*, double*, int64_t*);
int oracle_encode_keys(const void*, void*, int32_t, int64_t, int64_t, int64_t, int32_t, const int32_t*, double,
                       int32_t);
int oracle_kv_cosine(const void*, const void*, int32_t, int64_t, int64_t, double*, int32_t);

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static uint32_t rng = 12345u;
static float frand(void) {
  rng = rng * 1664525u + 1013904223u;
  return (float)((rng >> 8) & 0xffff) / 32768.0f - 1.0f;
}
static void fill(void* p, int32_t dtype, size_t n) {
  for (size_t i = 0; i < n; ++i) {
    const float v = frand();
    if (dtype == 1) {
      ((float*)p)[i] = v;
    } else {
      uint32_t u;
      memcpy(&u, &v, 4);
      ((uint16_t*)p)[i] = (uint16_t)(u >> 16);
    }
  }
}

int main(void) {
  /* rounding at special values */
  EXPECT(isnan(oracle_round_bf16(NAN)));
  EXPECT(isinf(oracle_round_bf16(INFINITY)));
  EXPECT(oracle_round_bf16(1e-45) == oracle_round_bf16(1e-45));
  EXPECT(oracle_round_bf16(0.0) == 0.0);

  for (int32_t dtype = 0; dtype <= 1; ++dtype) {
    const size_t es = dtype ? 4 : 2;
    const int32_t Ls = 3, Lt = 2, H = 2, D = 8, k = 2;
    const int64_t T = 5;
    oracle_problem pb = {Ls, Lt, H, D, k, dtype, 1, 2, T, 10000.0, 500000.0};
    void* sk = malloc(es * Ls * H * T * D);
    void* sv = malloc(es * Ls * H * T * D);
    void* wk = malloc(es * Lt * H * k * D * D);
    void* wv = malloc(es * Lt * H * k * D * D);
    float* bk = malloc(4 * Lt * H * D);
    float* bv = malloc(4 * Lt * H * D);
    fill(sk, dtype, (size_t)Ls * H * T * D);
    fill(sv, dtype, (size_t)Ls * H * T * D);
    fill(wk, dtype, (size_t)Lt * H * k * D * D);
    fill(wv, dtype, (size_t)Lt * H * k * D * D);
    fill(bk, 1, (size_t)Lt * H * D);
    fill(bv, 1, (size_t)Lt * H * D);
    int32_t spos[5] = {0, 7, -3, 100000, 2147483000}, tpos[5] = {4, 1, 0, -5, 99};
    int32_t sel[4] = {2, 0, 1, 1};
    const int64_t n_all = Lt * H * T;
    double* ok = malloc(sizeof(double) * n_all * D);
    double* ov = malloc(sizeof(double) * n_all * D);
    EXPECT(oracle_transfer_rows(&pb, sk, sv, spos, tpos, sel, wk, bk, wv, bv, 0, NULL, ok, ov) == 0);
    for (int64_t i = 0; i < n_all * D; ++i) EXPECT(isfinite(ok[i]) && isfinite(ov[i]));
    int64_t rows[3] = {0, n_all - 1, 7};
    EXPECT(oracle_transfer_rows(&pb, sk, sv, spos, tpos, sel, wk, bk, wv, bv, 3, rows, ok, ov) == 0);
    int64_t bad_rows[1] = {n_all};
    EXPECT(oracle_transfer_rows(&pb, sk, sv, spos, tpos, sel, wk, bk, wv, bv, 1, bad_rows, ok, ov) == 1);
    int32_t bad_sel[4] = {2, 3, 1, 1};
    EXPECT(oracle_transfer_rows(&pb, sk, sv, spos, tpos, bad_sel, wk, bk, wv, bv, 0, NULL, ok, ov) == 1);
    oracle_problem bad = pb;
    bad.head_dim = 7;
    EXPECT(oracle_transfer_rows(&bad, sk, sv, spos, tpos, sel, wk, bk, wv, bv, 0, NULL, ok, ov) == 1);

    /* wide map: IN = k * 2 * H * D */
    const int64_t IN = (int64_t)k * 2 * H * D;
    void* wwk = malloc(es * Lt * H * IN * D);
    void* wwv = malloc(es * Lt * H * IN * D);
    fill(wwk, dtype, (size_t)(Lt * H * IN * D));
    fill(wwv, dtype, (size_t)(Lt * H * IN * D));
    EXPECT(oracle_transfer_wide_rows(&pb, sk, sv, spos, tpos, sel, wwk, bk, wwv, bv, 0, NULL, ok, ov) == 0);
    EXPECT(oracle_transfer_wide_rows(&pb, sk, sv, spos, tpos, bad_sel, wwk, bk, wwv, bv, 0, NULL, ok, ov) == 1);

    /* paged: 2 requests of 3 and 2 tokens, block size 2 */
    oracle_paged pg = {2, 2, 2, 2, 4, 5};
    const int64_t slots_s = 4 * 2, slots_t = 5 * 2;
    void* pk = malloc(es * Ls * slots_s * H * D);
    void* pv = malloc(es * Ls * slots_s * H * D);
    fill(pk, dtype, (size_t)(Ls * slots_s * H * D));
    fill(pv, dtype, (size_t)(Ls * slots_s * H * D));
    int32_t sbt[4] = {3, 0, 1, 2}, tbt[4] = {4, 1, 0, 2}, cu[3] = {0, 3, 5};
    int64_t dst[8];
    const int64_t np = Lt * H * 5;
    EXPECT(oracle_transfer_paged_rows(&pb, &pg, pk, pv, sbt, tbt, cu, spos, tpos, sel, wk, bk, wv, bv, 0, NULL, ok,
                                      ov, NULL) == 0);
    int64_t prow[8] = {0, 1, 2, 3, 4, np - 1, np - 2, 9};
    EXPECT(oracle_transfer_paged_rows(&pb, &pg, pk, pv, sbt, tbt, cu, spos, tpos, sel, wk, bk, wv, bv, 8, prow, ok,
                                      ov, dst) == 0);
    int32_t bad_bt[4] = {3, 0, 9, 2};
    EXPECT(oracle_transfer_paged_rows(&pb, &pg, pk, pv, bad_bt, tbt, cu, spos, tpos, sel, wk, bk, wv, bv, 0, NULL,
                                      ok, ov, NULL) == 1);

    /* key encoding and the KV cosine */
    void* enc = malloc(es * Ls * H * T * D);
    EXPECT(oracle_encode_keys(sk, enc, dtype, Ls, H, T, D, spos, 10000.0, 2) == 0);
    EXPECT(oracle_encode_keys(sk, enc, dtype, Ls, H, T, 7, spos, 10000.0, 2) == 1);
    double cs[6];
    EXPECT(oracle_kv_cosine(sk, enc, dtype, 6, (int64_t)T * D, cs, 2) == 0);
    EXPECT(oracle_kv_cosine(sk, enc, 9, 6, (int64_t)T * D, cs, 2) == 1);

    free(sk); free(sv); free(wk); free(wv); free(bk); free(bv); free(ok); free(ov);
    free(wwk); free(wwv); free(pk); free(pv); free(enc);
  }
  if (failures) fprintf(stderr, "%d expectation(s) failed\n", failures);
  else printf("oracle driver: all calls as expected\n");
  return failures ? 1 : 0;
}
