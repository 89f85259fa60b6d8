/*
 * qsa_oracle.c -- reference CPU implementation of packed QSA decode.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the HIP path is
 * checked against.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load it; the product path never does.  It shares
 * no code, header, table or constant with the HIP library.
 *
 * What it computes (the plain definition, written out, in double precision):
 *
 *   Page "fix(qsa): restore SM121 correctness with Humanize and Kernel Design
 *   Agent" (sglang #36845), section "Changes": one query row per packed
 *   sequence, BF16, head dim 256, 12:1 GQA (24 Q heads over 2 KV heads, or 12
 *   over 1), at most 2055 selected KV entries per row, lengths read from
 *   cu_seqlens.  Section "Optimized kernel": softmax attention of each Q head
 *   over the K/V rows of its KV head; the split/merge and online softmax named
 *   there are re-associations of the same sum, so the oracle does none of it:
 *   it computes the two-pass textbook softmax directly.
 *
 *   Page "[Kernel][WIP] Integrate native FlashInfer SM70 batch GDN and QSA
 *   probes" (1Cat-vLLM #523), QSA description: the selected indices are read
 *   in list order and duplicates are kept, so a repeated slot is counted
 *   every time it is listed.
 *
 *   Page "feat(qsa): quantized KV pools with dequant-on-gather
 *   (fp8/int8/int4)" (sglang #37798), part 4 "Modifications": the fp8 pool
 *   holds e4m3fn bytes; the int8 pool holds signed codes times a scale per
 *   channel group; the int4 pool packs two codes per byte, the low nibble
 *   holding the even channel, stored offset-binary (q + 8), times a scale per
 *   32-channel group.  Dequantization is code value times its group scale.
 *
 *   Same page and section, tiered pool bullet: every token is written to an
 *   int8 ring of R rows (R a power of two, one fp16 scale per 64 channels)
 *   and to the full int4 pool (one fp16 scale per 32 channels), and an int32
 *   owner table records which slot each ring row holds; a reader takes the
 *   ring row r = slot & (R - 1) when owner[r] == slot and the int4 row
 *   otherwise.  oracle_qsa_decode_tiered makes that choice per listed entry.
 *
 * Readings where the pages are silent (each one is listed in the design
 * notes): the softmax scale is 1/sqrt(256) = 1/16; Q head h uses KV head
 * h / 12; lse is the natural log of the sum of exp over the scaled logits;
 * a zero-length row gives o = 0 and lse = -inf; the fp8 pool carries a
 * scale too (per row in the measured configuration) that multiplies the
 * decoded e4m3fn value.
 *
 * Arithmetic: every operand is widened exactly to double; dot products,
 * exponentials and sums run in double in list order.  The outputs are
 * returned in double; the caller compares the GPU's bf16/fp32 outputs to
 * them.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* KV formats (oracle's own numbering). */
enum { ORC_BF16 = 0, ORC_FP8_E4M3FN = 1, ORC_INT8 = 2, ORC_INT4 = 3 };

/* Error codes returned by oracle_qsa_decode. */
enum {
  ORC_OK = 0,
  ORC_BAD_ARGS = 1,   /* shapes, format or group size outside the contract */
  ORC_BAD_CU = 2,     /* cu_seqlens not a valid packing of sel */
  ORC_BAD_LEN = 3,    /* a row longer than the capacity */
  ORC_BAD_SLOT = 4,   /* a selected slot outside [0, slots) */
};

#define ORC_HEAD_DIM 256
#define ORC_GQA 12
#define ORC_CAPACITY 2055

/* bf16 -> double: a bf16 value is the upper 16 bits of an IEEE binary32. */
static double bf16_to_double(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP e4m3fn -> double, from the format's definition: 1 sign bit, 4 exponent
 * bits with bias 7, 3 mantissa bits; exponent field 0 is subnormal
 * (m * 2^-9); the only NaN encodings are S.1111.111; there is no infinity. */
double oracle_fp8_e4m3fn_to_double(uint8_t code) {
  int sign = (code >> 7) & 1;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double v;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -v : v;
}

/* Bytes used by one (slot, kv-head) row's codes in each format. */
static int64_t row_code_bytes(int fmt) {
  switch (fmt) {
    case ORC_BF16: return 2 * ORC_HEAD_DIM;
    case ORC_FP8_E4M3FN: return ORC_HEAD_DIM;
    case ORC_INT8: return ORC_HEAD_DIM;
    case ORC_INT4: return ORC_HEAD_DIM / 2;
    default: return -1;
  }
}

/* Dequantize one (slot, kv-head) row to double.
 *   pool  : [slots][hkv][row_code_bytes] contiguous codes
 *   scale : [slots][hkv][256/group] fp32 (unused for bf16) */
void oracle_dequant_row(int fmt, int group, int hkv, const void *pool,
                        const float *scale, int64_t slot, int g,
                        double *out /* [256] */) {
  int64_t rb = row_code_bytes(fmt);
  const uint8_t *row = (const uint8_t *)pool + (slot * hkv + g) * rb;
  int ngroups = (fmt == ORC_BF16) ? 0 : ORC_HEAD_DIM / group;
  const float *sc = (fmt == ORC_BF16) ? NULL : scale + (slot * hkv + g) * ngroups;
  for (int d = 0; d < ORC_HEAD_DIM; ++d) {
    double code;
    switch (fmt) {
      case ORC_BF16: {
        uint16_t bits;
        memcpy(&bits, row + 2 * d, 2);
        out[d] = bf16_to_double(bits);
        continue;
      }
      case ORC_FP8_E4M3FN:
        code = oracle_fp8_e4m3fn_to_double(row[d]);
        break;
      case ORC_INT8:
        code = (double)(int8_t)row[d];
        break;
      case ORC_INT4: {
        uint8_t byte = row[d / 2];
        int nib = (d % 2 == 0) ? (byte & 0xF) : (byte >> 4);
        code = (double)(nib - 8);
        break;
      }
      default:
        code = NAN;
    }
    out[d] = code * (double)sc[d / group];
  }
}

/* Check cu_seqlens / sel against the contract.  Returns an ORC_* code. */
static int check_packing(int bs, const int32_t *cu, int64_t n_sel,
                         const int32_t *sel, int64_t slots) {
  for (int b = 0; b < bs; ++b) {
    if (cu[b] < 0 || cu[b + 1] < cu[b] || (int64_t)cu[b + 1] > n_sel) return ORC_BAD_CU;
    if (cu[b + 1] - cu[b] > ORC_CAPACITY) return ORC_BAD_LEN;
    for (int32_t i = cu[b]; i < cu[b + 1]; ++i)
      if (sel[i] < 0 || (int64_t)sel[i] >= slots) return ORC_BAD_SLOT;
  }
  return ORC_OK;
}

/* Where the K and V rows of a listed slot come from: one pool, or the
 * tiered pair (int8 ring + int4 pool with an owner table). */
struct kv_source {
  int tiered;
  int hkv;
  /* single pool (tiered: the int4 pool) */
  int fmt, group;
  const void *k_pool, *v_pool;
  const float *k_scale, *v_scale;
  /* tiered: ring of R rows */
  int64_t ring_rows;
  const int32_t *owner;
  const void *ring_k, *ring_v;
  const float *ring_k_scale, *ring_v_scale;
};

/* The dequantized K (is_v = 0) or V (is_v = 1) row of (slot, kv head g). */
static void fetch_row(const struct kv_source *src, int is_v, int64_t slot, int g, double *out) {
  if (src->tiered) {
    const int64_t r = slot & (src->ring_rows - 1);
    if (src->owner[r] == slot) {
      oracle_dequant_row(ORC_INT8, 64, src->hkv, is_v ? src->ring_v : src->ring_k,
                         is_v ? src->ring_v_scale : src->ring_k_scale, r, g, out);
      return;
    }
    oracle_dequant_row(ORC_INT4, 32, src->hkv, is_v ? src->v_pool : src->k_pool,
                       is_v ? src->v_scale : src->k_scale, slot, g, out);
    return;
  }
  oracle_dequant_row(src->fmt, src->group, src->hkv, is_v ? src->v_pool : src->k_pool,
                     is_v ? src->v_scale : src->k_scale, slot, g, out);
}

/* Two-pass softmax attention of every (row, Q head) over its listed rows. */
static void attend(int bs, int hq, const uint16_t *q, const struct kv_source *src,
                   const int32_t *sel, const int32_t *cu, double sm_scale, double *out,
                   double *lse, int nthreads) {
  const int npairs = bs * hq;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
  for (int pair = 0; pair < npairs; ++pair) {
    const int b = pair / hq;
    const int h = pair % hq;
    const int g = h / ORC_GQA;
    const int32_t begin = cu[b];
    const int32_t len = cu[b + 1] - cu[b];
    double *o = out + ((int64_t)b * hq + h) * ORC_HEAD_DIM;

    double qv[ORC_HEAD_DIM];
    for (int d = 0; d < ORC_HEAD_DIM; ++d)
      qv[d] = bf16_to_double(q[((int64_t)b * hq + h) * ORC_HEAD_DIM + d]);

    if (len == 0) { /* empty sum: o = 0, lse = log(0) */
      for (int d = 0; d < ORC_HEAD_DIM; ++d) o[d] = 0.0;
      lse[(int64_t)b * hq + h] = -INFINITY;
      continue;
    }

    /* pass 1: logits s_j = sm_scale * sum_d q[d] * K_j[d], list order */
    double *s = (double *)malloc(sizeof(double) * (size_t)len);
    double row[ORC_HEAD_DIM];
    double m = -INFINITY;
    for (int32_t j = 0; j < len; ++j) {
      fetch_row(src, 0, sel[begin + j], g, row);
      double dot = 0.0;
      for (int d = 0; d < ORC_HEAD_DIM; ++d) dot += qv[d] * row[d];
      s[j] = dot * sm_scale;
      if (s[j] > m) m = s[j];
    }

    /* pass 2: p_j = exp(s_j - m), l = sum p_j, o = sum p_j V_j / l */
    double l = 0.0;
    double acc[ORC_HEAD_DIM];
    for (int d = 0; d < ORC_HEAD_DIM; ++d) acc[d] = 0.0;
    for (int32_t j = 0; j < len; ++j) {
      double p = exp(s[j] - m);
      l += p;
      fetch_row(src, 1, sel[begin + j], g, row);
      for (int d = 0; d < ORC_HEAD_DIM; ++d) acc[d] += p * row[d];
    }
    for (int d = 0; d < ORC_HEAD_DIM; ++d) o[d] = acc[d] / l;
    lse[(int64_t)b * hq + h] = m + log(l);
    free(s);
  }
}

/*
 * oracle_qsa_decode
 *   q        [bs][hq][256] bf16 bits, contiguous
 *   k_pool   [slots][hkv][row bytes] codes, contiguous (same for v_pool)
 *   k_scale  [slots][hkv][256/group] fp32 (NULL for bf16; same for v_scale)
 *   sel      [n_sel] int32 slot ids; row b uses sel[cu[b] .. cu[b+1])
 *   cu       [bs+1] int32
 *   sm_scale softmax scale applied to q.k (1/16 for head dim 256)
 *   out      [bs][hq][256] double, written
 *   lse      [bs][hq] double, written (natural log)
 *   nthreads OpenMP threads over (row, head) pairs; <= 0 means 1
 */
int oracle_qsa_decode(int bs, int hq, int hkv, const uint16_t *q, int fmt,
                      int group, int64_t slots, const void *k_pool,
                      const void *v_pool, const float *k_scale,
                      const float *v_scale, const int32_t *sel, int64_t n_sel,
                      const int32_t *cu, double sm_scale, double *out,
                      double *lse, int nthreads) {
  if (bs < 1 || hkv < 1 || hq != ORC_GQA * hkv || slots < 1) return ORC_BAD_ARGS;
  if (row_code_bytes(fmt) < 0) return ORC_BAD_ARGS;
  if (fmt != ORC_BF16) {
    if (group < 1 || ORC_HEAD_DIM % group != 0 || !k_scale || !v_scale) return ORC_BAD_ARGS;
    if (fmt == ORC_INT4 && group % 2 != 0) return ORC_BAD_ARGS;
  }
  int rc = check_packing(bs, cu, n_sel, sel, slots);
  if (rc != ORC_OK) return rc;
  if (nthreads < 1) nthreads = 1;
  struct kv_source src = {0};
  src.hkv = hkv;
  src.fmt = fmt;
  src.group = group;
  src.k_pool = k_pool;
  src.v_pool = v_pool;
  src.k_scale = k_scale;
  src.v_scale = v_scale;
  attend(bs, hq, q, &src, sel, cu, sm_scale, out, lse, nthreads);
  return ORC_OK;
}

/*
 * oracle_qsa_decode_tiered -- same contract, rows from a tiered pool:
 *   ring_k / ring_v   [ring_rows][hkv][256] int8 codes
 *   ring_k_scale ...  [ring_rows][hkv][4] fp32 (the fp16 scales' values)
 *   owner             [ring_rows] int32
 *   cold_k / cold_v   [slots][hkv][128] int4 pairs
 *   cold_k_scale ...  [slots][hkv][8] fp32 (the fp16 scales' values)
 * ring_rows must be a power of two.
 */
int oracle_qsa_decode_tiered(int bs, int hq, int hkv, const uint16_t *q, int64_t ring_rows,
                             const int32_t *owner, const void *ring_k, const void *ring_v,
                             const float *ring_k_scale, const float *ring_v_scale,
                             int64_t slots, const void *cold_k, const void *cold_v,
                             const float *cold_k_scale, const float *cold_v_scale,
                             const int32_t *sel, int64_t n_sel, const int32_t *cu,
                             double sm_scale, double *out, double *lse, int nthreads) {
  if (bs < 1 || hkv < 1 || hq != ORC_GQA * hkv || slots < 1) return ORC_BAD_ARGS;
  if (ring_rows < 1 || (ring_rows & (ring_rows - 1)) != 0) return ORC_BAD_ARGS;
  if (!owner || !ring_k || !ring_v || !ring_k_scale || !ring_v_scale || !cold_k || !cold_v ||
      !cold_k_scale || !cold_v_scale)
    return ORC_BAD_ARGS;
  int rc = check_packing(bs, cu, n_sel, sel, slots);
  if (rc != ORC_OK) return rc;
  if (nthreads < 1) nthreads = 1;
  struct kv_source src = {0};
  src.tiered = 1;
  src.hkv = hkv;
  src.k_pool = cold_k;
  src.v_pool = cold_v;
  src.k_scale = cold_k_scale;
  src.v_scale = cold_v_scale;
  src.ring_rows = ring_rows;
  src.owner = owner;
  src.ring_k = ring_k;
  src.ring_v = ring_v;
  src.ring_k_scale = ring_k_scale;
  src.ring_v_scale = ring_v_scale;
  attend(bs, hq, q, &src, sel, cu, sm_scale, out, lse, nthreads);
  return ORC_OK;
}

/* Number of OpenMP threads a parallel region with this request actually gets. */
int oracle_threads_used(int nthreads) {
#ifdef _OPENMP
  int used = 1;
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel num_threads(nthreads)
  {
#pragma omp single
    used = omp_get_num_threads();
  }
  return used;
#else
  (void)nthreads;
  return 1;
#endif
}
