/*
 * qsa_index_oracle.c -- reference CPU implementation of the QSA indexer step
 * that produces the decode's selected slot lists.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load it; the product path never
 * does.  It shares no code, header, table or constant with the HIP library.
 *
 * What the pages fix:
 *
 *   Page "[Kernel][WIP] Integrate native FlashInfer SM70 batch GDN and QSA
 *   probes" (1Cat-vLLM #523), follow-up "device-planned MQA and QSA quality
 *   attribution": the indexer is MQA scoring, an exact top-k and an index
 *   expansion, with a fixed 256K-token capacity.
 *
 *   Page "feat(qsa): quantized KV pools with dequant-on-gather
 *   (fp8/int8/int4)", part 4, decode routing paragraph: the index row is
 *   token_topk + compress_ratio - 1 entries wide (2051 for a budget of 2048
 *   tokens and a compression ratio of 4).
 *
 * Reading taken where the pages are silent (listed in the design notes):
 *
 *   Row b has T_b context tokens; logical block j (0 <= j < n_b = T_b / c)
 *   covers tokens j*c .. j*c + c - 1 and has one compressed index key,
 *   stored in pool row block_table[b][j].  MQA scoring: the row's hi index
 *   query heads share that key, and block j scores
 *       s_j = sum_h w_h * (q_h . k_j) = (sum_h w_h q_h) . k_j
 *   (w_h = 1 when no weights are given), evaluated in fp32 exactly as
 *   written below: the row's weighted query qt = sum_h w_h q_h first,
 *   element by element, one fused multiply-add per head in head order
 *   starting from 0; then the dot product qt . k_j, one fused multiply-add
 *   per element in element order starting from 0; -0 is read as +0.  Both
 *   this oracle and the GPU evaluate it in that order, so they take the
 *   same top-k decisions.
 *
 *   Exact top-k: the K = budget / c blocks with the largest scores, a tie
 *   going to the lower block index; with n_b <= K every block is taken.
 *
 *   Expansion: the taken blocks in ascending block order, each giving its c
 *   tokens in order, then the T_b mod c newest tokens (those not yet in a
 *   complete block).  A row therefore lists min(n_b, K) * c + T_b mod c
 *   tokens (at most budget + c - 1), in ascending logical position, and
 *   every token t becomes the KV slot req_to_token[b][t].  Rows are packed
 *   one after another; cu receives the offsets.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static float bf16_to_float(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* The row's weighted query qt[d] = sum_h w_h q[h][d] of the reading above. */
static void weighted_query(int hi, int di, const uint16_t *q, const float *w, float *qt) {
  for (int d = 0; d < di; ++d) {
    float a = 0.0f;
    for (int h = 0; h < hi; ++h) a = fmaf(w ? w[h] : 1.0f, bf16_to_float(q[h * di + d]), a);
    qt[d] = a;
  }
}

/* Block score of the reading above: qt . k in element order. */
static float block_score(int di, const float *qt, const uint16_t *k) {
  float s = 0.0f;
  for (int d = 0; d < di; ++d) s = fmaf(qt[d], bf16_to_float(k[d]), s);
  return s + 0.0f; /* -0 -> +0 */
}

struct scored {
  float s;
  int32_t j;
};

/* larger score first; equal scores: lower block index first */
static int by_score(const void *pa, const void *pb) {
  const struct scored *a = pa, *b = pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->j > b->j) - (a->j < b->j);
}

static int by_index(const void *pa, const void *pb) {
  const int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
  return (a > b) - (a < b);
}

/* Tokens a row lists, from its context length alone. */
static int64_t row_length(int64_t t, int budget, int c) {
  const int64_t n = t / c, k = budget / c;
  return (n < k ? n : k) * c + t % c;
}

/*
 * Returns 0, or 1 bad arguments, 5 a context length outside
 * [0, max_tokens] or with more blocks than max_blocks, 6 a block table
 * entry outside [0, n_kpool).  scores_out ([bs][max_blocks], may be NULL)
 * receives every block's score (entries past n_b untouched).
 */
int oracle_qsa_index(int bs, int hi, int di, const uint16_t *q, const float *w,
                     const uint16_t *kpool, int64_t n_kpool, const int32_t *block_table,
                     int max_blocks, const int32_t *req_to_token, int max_tokens,
                     const int32_t *ctx_len, int budget, int c, int32_t *sel_out, int32_t *cu_out,
                     float *scores_out) {
  if (bs < 1 || hi < 1 || di < 1 || c < 1 || budget < c || budget % c || !q || !kpool ||
      !block_table || !req_to_token || !ctx_len || !sel_out || !cu_out)
    return 1;
  cu_out[0] = 0;
  for (int b = 0; b < bs; ++b) {
    const int64_t t = ctx_len[b];
    if (t < 0 || t > max_tokens || t / c > max_blocks) return 5;
    cu_out[b + 1] = (int32_t)(cu_out[b] + row_length(t, budget, c));
  }
  for (int b = 0; b < bs; ++b) {
    const int64_t t = ctx_len[b];
    const int n = (int)(t / c), k = budget / c;
    struct scored *sc = malloc(sizeof *sc * (n > 0 ? n : 1));
    int32_t *take = malloc(sizeof *take * (n > 0 ? n : 1));
    if (!sc || !take) {
      free(sc);
      free(take);
      return 1;
    }
    float *qt = malloc(sizeof *qt * (size_t)di);
    if (!qt) {
      free(sc);
      free(take);
      return 1;
    }
    weighted_query(hi, di, q + (int64_t)b * hi * di, w ? w + (int64_t)b * hi : NULL, qt);
    for (int j = 0; j < n; ++j) {
      const int32_t row = block_table[(int64_t)b * max_blocks + j];
      if (row < 0 || row >= n_kpool) {
        free(sc);
        free(take);
        free(qt);
        return 6;
      }
      sc[j].s = block_score(di, qt, kpool + (int64_t)row * di);
      sc[j].j = j;
      if (scores_out) scores_out[(int64_t)b * max_blocks + j] = sc[j].s;
    }
    int ntake = n;
    if (n > k) {
      qsort(sc, (size_t)n, sizeof *sc, by_score);
      ntake = k;
    }
    for (int i = 0; i < ntake; ++i) take[i] = sc[i].j;
    qsort(take, (size_t)ntake, sizeof *take, by_index);
    int32_t *out = sel_out + cu_out[b];
    const int32_t *r2t = req_to_token + (int64_t)b * max_tokens;
    int64_t o = 0;
    for (int i = 0; i < ntake; ++i)
      for (int e = 0; e < c; ++e) out[o++] = r2t[(int64_t)take[i] * c + e];
    for (int64_t pos = (int64_t)n * c; pos < t; ++pos) out[o++] = r2t[pos];
    free(sc);
    free(take);
    free(qt);
  }
  return 0;
}
