/* oracle_check.c -- drives every entry point of the C oracle in a process
 * built with AddressSanitizer and UndefinedBehaviorSanitizer: small random
 * calls in every pool format, the tiered reader, the indexer and the
 * rejection paths, with a few closed-form checks (a single entry returns
 * its V row, an empty row gives 0 and -inf).  Exit status 0 when every
 * expectation holds. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_fp8_e4m3fn_to_double(uint8_t code);
void oracle_dequant_row(int fmt, int group, int hkv, const void *pool, const float *scale,
                        int64_t slot, int g, double *out);
int oracle_qsa_decode(int bs, int hq, int hkv, const uint16_t *q, int fmt, int group,
                      int64_t slots, const void *k_pool, const void *v_pool, const float *k_scale,
                      const float *v_scale, const int32_t *sel, int64_t n_sel, const int32_t *cu,
                      double sm_scale, double *out, double *lse, int nthreads);
int oracle_qsa_decode_tiered(int bs, int hq, int hkv, const uint16_t *q, int64_t ring_rows,
                             const int32_t *owner, const void *ring_k, const void *ring_v,
                             const float *ring_k_scale, const float *ring_v_scale, int64_t slots,
                             const void *cold_k, const void *cold_v, const float *cold_k_scale,
                             const float *cold_v_scale, const int32_t *sel, int64_t n_sel,
                             const int32_t *cu, double sm_scale, double *out, double *lse,
                             int nthreads);
int oracle_qsa_index(int bs, int hi, int di, const uint16_t *q, const float *w,
                     const uint16_t *kpool, int64_t n_kpool, const int32_t *block_table,
                     int max_blocks, const int32_t *req_to_token, int max_tokens,
                     const int32_t *ctx_len, int budget, int c, int32_t *sel_out, int32_t *cu_out,
                     float *scores_out);
int oracle_threads_used(int nthreads);

static int g_fail = 0;
#define EXPECT(cond, ...)                                   \
  do {                                                      \
    if (!(cond)) {                                          \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);  \
      fprintf(stderr, __VA_ARGS__);                         \
      fprintf(stderr, "\n");                                \
      ++g_fail;                                             \
    }                                                       \
  } while (0)

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) { /* xorshift64*: test data only */
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return (uint32_t)((g_state * 0x2545F4914F6CDD1Dull) >> 32);
}
/* a finite bf16 in about [-4, 4) */
static uint16_t rand_bf16(void) {
  const uint32_t sign = next_u32() & 1u, exp = 125u + next_u32() % 4u, man = next_u32() & 0x7Fu;
  return (uint16_t)((sign << 15) | (exp << 7) | man);
}

static void *xmalloc(size_t n) {
  void *p = malloc(n ? n : 1);
  if (!p) exit(3);
  return p;
}

static void decode_formats(void) {
  enum { BS = 3, HKV = 2, HQ = 24, SLOTS = 40, D = 256 };
  const int lens[BS] = {5, 0, 37};
  int32_t cu[BS + 1] = {0};
  for (int b = 0; b < BS; ++b) cu[b + 1] = cu[b] + lens[b];
  const int n_sel = cu[BS];
  int32_t *sel = xmalloc(sizeof(int32_t) * n_sel);
  for (int i = 0; i < n_sel; ++i) sel[i] = (int32_t)(next_u32() % SLOTS);
  sel[1] = sel[0]; /* a duplicate */
  uint16_t *q = xmalloc(sizeof(uint16_t) * BS * HQ * D);
  for (int i = 0; i < BS * HQ * D; ++i) q[i] = rand_bf16();
  double *out = xmalloc(sizeof(double) * BS * HQ * D), *lse = xmalloc(sizeof(double) * BS * HQ);
  const int fmts[4] = {0, 1, 2, 3}, row_bytes[4] = {512, 256, 256, 128};
  const int groups[4] = {256, 64, 256, 32};
  for (int f = 0; f < 4; ++f) {
    const size_t pool_bytes = (size_t)SLOTS * HKV * row_bytes[f];
    uint8_t *k = xmalloc(pool_bytes), *v = xmalloc(pool_bytes);
    for (size_t i = 0; i < pool_bytes; ++i) {
      k[i] = (uint8_t)next_u32();
      v[i] = (uint8_t)next_u32();
    }
    if (f == 0) /* finite bf16 values */
      for (size_t i = 0; i < pool_bytes / 2; ++i) {
        ((uint16_t *)k)[i] = rand_bf16();
        ((uint16_t *)v)[i] = rand_bf16();
      }
    if (f == 1) /* no NaN codes */
      for (size_t i = 0; i < pool_bytes; ++i) {
        if ((k[i] & 0x7F) == 0x7F) k[i] ^= 1;
        if ((v[i] & 0x7F) == 0x7F) v[i] ^= 1;
      }
    const int ng = D / groups[f];
    float *ks = xmalloc(sizeof(float) * SLOTS * HKV * ng), *vs = xmalloc(sizeof(float) * SLOTS * HKV * ng);
    for (int i = 0; i < SLOTS * HKV * ng; ++i) {
      ks[i] = 0.01f + (float)(next_u32() % 100) / 1000.0f;
      vs[i] = 0.01f + (float)(next_u32() % 100) / 1000.0f;
    }
    const int rc = oracle_qsa_decode(BS, HQ, HKV, q, fmts[f], groups[f], SLOTS, k, v, f ? ks : NULL,
                                     f ? vs : NULL, sel, n_sel, cu, 1.0 / 16.0, out, lse, 2);
    EXPECT(rc == 0, "decode fmt %d rc %d", f, rc);
    for (int h = 0; h < HQ; ++h) {
      EXPECT(isinf(lse[1 * HQ + h]) && lse[1 * HQ + h] < 0, "empty row lse");
      for (int d = 0; d < D; ++d) EXPECT(out[(1 * HQ + h) * D + d] == 0.0, "empty row out");
    }
    for (int i = 0; i < BS * HQ * D; ++i) EXPECT(isfinite(out[i]) || (i / (HQ * D)) == 1, "finite out");
    /* a single entry returns that V row */
    int32_t one_cu[2] = {0, 1};
    double row[D];
    EXPECT(oracle_qsa_decode(1, HQ, HKV, q, fmts[f], groups[f], SLOTS, k, v, f ? ks : NULL, f ? vs : NULL,
                             sel + 2, 1, one_cu, 1.0 / 16.0, out, lse, 1) == 0, "single entry");
    for (int g = 0; g < HKV; ++g) {
      oracle_dequant_row(fmts[f], groups[f], HKV, v, vs, sel[2], g, row);
      for (int h = 12 * g; h < 12 * g + 12; ++h)
        for (int d = 0; d < D; ++d) EXPECT(out[h * D + d] == row[d], "single entry = V row");
    }
    /* rejections */
    int32_t bad_cu[BS + 1] = {0, 3, 2, 5};
    EXPECT(oracle_qsa_decode(BS, HQ, HKV, q, fmts[f], groups[f], SLOTS, k, v, ks, vs, sel, n_sel, bad_cu,
                             1.0 / 16.0, out, lse, 1) == 2, "bad cu");
    sel[0] = SLOTS;
    EXPECT(oracle_qsa_decode(BS, HQ, HKV, q, fmts[f], groups[f], SLOTS, k, v, ks, vs, sel, n_sel, cu,
                             1.0 / 16.0, out, lse, 1) == 4, "bad slot");
    sel[0] = 0;
    EXPECT(oracle_qsa_decode(BS, 12, HKV, q, fmts[f], groups[f], SLOTS, k, v, ks, vs, sel, n_sel, cu,
                             1.0 / 16.0, out, lse, 1) == 1, "bad heads");
    free(k);
    free(v);
    free(ks);
    free(vs);
  }
  /* a row longer than 2055 */
  int32_t *long_sel = xmalloc(sizeof(int32_t) * 2056);
  memset(long_sel, 0, sizeof(int32_t) * 2056);
  int32_t long_cu[2] = {0, 2056};
  uint16_t *pool = xmalloc(sizeof(uint16_t) * SLOTS * HKV * D);
  memset(pool, 0, sizeof(uint16_t) * SLOTS * HKV * D);
  EXPECT(oracle_qsa_decode(1, HQ, HKV, q, 0, 256, SLOTS, pool, pool, NULL, NULL, long_sel, 2056, long_cu,
                           1.0 / 16.0, out, lse, 1) == 3, "row > 2055");
  free(long_sel);
  free(pool);
  for (int c = 0; c < 256; ++c) {
    const double x = oracle_fp8_e4m3fn_to_double((uint8_t)c);
    EXPECT(((c & 0x7F) == 0x7F) ? isnan(x) : (isfinite(x) && fabs(x) <= 448.0), "fp8 code %d", c);
  }
  free(sel);
  free(q);
  free(out);
  free(lse);
}

static void decode_tiered(void) {
  enum { BS = 2, HKV = 1, HQ = 12, SLOTS = 300, R = 64, D = 256 };
  int32_t cu[BS + 1] = {0, 50, 120};
  int32_t sel[120];
  for (int i = 0; i < 120; ++i) sel[i] = (int32_t)(next_u32() % SLOTS);
  int32_t owner[R];
  for (int r = 0; r < R; ++r) owner[r] = (r % 3 == 0) ? -1 : r + R * (int)(next_u32() % 4);
  int8_t *rk = xmalloc(R * HKV * D), *rv = xmalloc(R * HKV * D);
  uint8_t *ck = xmalloc(SLOTS * HKV * D / 2), *cv = xmalloc(SLOTS * HKV * D / 2);
  for (int i = 0; i < R * HKV * D; ++i) {
    rk[i] = (int8_t)next_u32();
    rv[i] = (int8_t)next_u32();
  }
  for (int i = 0; i < SLOTS * HKV * D / 2; ++i) {
    ck[i] = (uint8_t)next_u32();
    cv[i] = (uint8_t)next_u32();
  }
  float rks[R * HKV * 4], rvs[R * HKV * 4], *cks = xmalloc(sizeof(float) * SLOTS * HKV * 8),
        *cvs = xmalloc(sizeof(float) * SLOTS * HKV * 8);
  for (int i = 0; i < R * HKV * 4; ++i) rks[i] = rvs[i] = 0.02f;
  for (int i = 0; i < SLOTS * HKV * 8; ++i) cks[i] = cvs[i] = 0.15f;
  uint16_t q[BS * HQ * D];
  for (int i = 0; i < BS * HQ * D; ++i) q[i] = rand_bf16();
  double *out = xmalloc(sizeof(double) * BS * HQ * D), lse[BS * HQ];
  EXPECT(oracle_qsa_decode_tiered(BS, HQ, HKV, q, R, owner, rk, rv, rks, rvs, SLOTS, ck, cv, cks, cvs, sel,
                                  120, cu, 1.0 / 16.0, out, lse, 2) == 0, "tiered decode");
  for (int i = 0; i < BS * HQ; ++i) EXPECT(isfinite(lse[i]), "tiered lse finite");
  EXPECT(oracle_qsa_decode_tiered(BS, HQ, HKV, q, 48, owner, rk, rv, rks, rvs, SLOTS, ck, cv, cks, cvs, sel,
                                  120, cu, 1.0 / 16.0, out, lse, 1) == 1, "ring of 48 rows");
  free(rk);
  free(rv);
  free(ck);
  free(cv);
  free(cks);
  free(cvs);
  free(out);
}

static void index_step(void) {
  enum { BS = 3, HI = 4, DI = 64, C = 4, BUDGET = 16, MAXT = 130, MAXB = MAXT / C + 1 };
  const int32_t ctx[BS] = {130, 0, 3};
  uint16_t q[BS * HI * DI], kpool[BS * MAXB * DI];
  for (int i = 0; i < BS * HI * DI; ++i) q[i] = rand_bf16();
  for (int i = 0; i < BS * MAXB * DI; ++i) kpool[i] = rand_bf16();
  float w[BS * HI];
  for (int i = 0; i < BS * HI; ++i) w[i] = 0.5f + (float)(next_u32() % 100) / 100.0f;
  int32_t bt[BS * MAXB], r2t[BS * MAXT];
  for (int i = 0; i < BS * MAXB; ++i) bt[i] = i;
  for (int i = 0; i < BS * MAXT; ++i) r2t[i] = (int32_t)(next_u32() % 100000);
  int32_t sel[BS * (BUDGET + C - 1) + 1], cu[BS + 1];
  float scores[BS * MAXB];
  EXPECT(oracle_qsa_index(BS, HI, DI, q, w, kpool, BS * MAXB, bt, MAXB, r2t, MAXT, ctx, BUDGET, C, sel, cu,
                          scores) == 0, "index");
  EXPECT(cu[0] == 0 && cu[1] == BUDGET + 130 % C && cu[2] == cu[1] && cu[3] == cu[2] + 3, "index cu");
  EXPECT(oracle_qsa_index(BS, HI, DI, q, NULL, kpool, BS * MAXB, bt, MAXB, r2t, MAXT, ctx, BUDGET, C, sel, cu,
                          NULL) == 0, "index without weights");
  bt[0] = -1;
  EXPECT(oracle_qsa_index(BS, HI, DI, q, w, kpool, BS * MAXB, bt, MAXB, r2t, MAXT, ctx, BUDGET, C, sel, cu,
                          NULL) == 6, "bad block table entry");
  bt[0] = 0;
  const int32_t bad_ctx[BS] = {MAXT + 1, 0, 0};
  EXPECT(oracle_qsa_index(BS, HI, DI, q, w, kpool, BS * MAXB, bt, MAXB, r2t, MAXT, bad_ctx, BUDGET, C, sel,
                          cu, NULL) == 5, "context too long");
  EXPECT(oracle_qsa_index(BS, HI, DI, q, w, kpool, BS * MAXB, bt, MAXB, r2t, MAXT, ctx, 15, C, sel, cu,
                          NULL) == 1, "budget not a multiple");
}

int main(void) {
  decode_formats();
  decode_tiered();
  index_step();
  EXPECT(oracle_threads_used(2) >= 1, "threads");
  printf("oracle_check: %s (%d failures)\n", g_fail ? "FAILED" : "ok", g_fail);
  return g_fail ? 1 : 0;
}
