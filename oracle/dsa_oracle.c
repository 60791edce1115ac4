/*
 * Plain CPU oracle for the DSA hot path: lightning-indexer scores, exact top-k,
 * and absorbed-MLA attention over the kept latent rows.
 *
 * TEST INFRASTRUCTURE ONLY.  This file exists so that tests, the smoke check and
 * the benchmark's CPU baseline have an independent answer to compare against.
 * It shares no code, header, table or constant with the HIP library, and the
 * library never calls it.  Everything here is computed in double precision with
 * plain loops, in the order the method states; OpenMP only spreads independent
 * queries or tokens across host threads.
 *
 * Sources (titles of the pages the method is described on):
 *   [GLM-A100] "GLM on an A100, in Vx", sections "The model" (what DSA computes:
 *              latent K/V per token, an indexer scoring every earlier token, the
 *              best 2,048 kept, everything kept below 2,048 tokens), "How do we
 *              know it is right?" (ReLU per indexer head before the heads are
 *              combined; ties resolved as a stable descending argsort), and
 *              "INT4, FP8 and BF16" (BF16 decoded exactly from exponent and
 *              mantissa; FP8 E4M3 with float32 scales).
 *   [glm-vx]   "Self-contained GLM-5 serving stack", component list (absorbed MLA
 *              decode, compressed request-local KV, stable softmax, FP8 E4M3FN
 *              decoding) and GPU section (split online-softmax compressed MLA).
 *
 * Readings where the pages leave a step open:
 *   - score[s] = sum_h w[h] * max(0, sum_d q[h][d] * khat[s][d]); one key row per
 *     token shared by all indexer heads; no extra scale inside the indexer.
 *   - fp8 keys: khat = e4m3fn(byte) * scale[token] (float32 per-token scale).
 *   - a query that sees n tokens (its own included) scores tokens 0..n-1.
 *   - top-k = first min(k, n) entries of a stable argsort of -score; NaN sorts
 *     after every number, -0.0 equals +0.0.  Kept indices are returned in
 *     ascending index order (order 0) or in that argsort order (order 1);
 *     unused slots hold -1.
 *   - absorbed MLA: the key is the whole latent row (kv_lora + rope wide), the
 *     value is its first kv_lora entries; lse is the natural-log sum-exp of the
 *     scaled logits.  No kept row: output 0, lse = -inf.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* dtype codes used by this oracle's own interface */
#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_E4M3FN 2

/* A token cache as the oracle reads it.  Token t of sequence b lives in
 * physical block p = block_table ? block_table[b * max_blocks + t / block_size] : b
 * at byte offset p * block_stride + (t % block_size) * row_stride from rows.
 * For fp8 rows the per-token scale is scale[p * scale_block_stride + t % block_size]. */
typedef struct {
  const uint8_t *rows;
  const float *scale;
  int64_t row_stride;
  int64_t block_stride;
  int64_t scale_block_stride;
  const int32_t *block_table;
  int32_t block_size;
  int32_t max_blocks;
  int32_t width;
  int32_t dtype;
} oracle_cache;

/* ---------------------------------------------------------------- codecs -- */

/* bf16: sign, 8-bit exponent with bias 127, 7-bit mantissa ([GLM-A100],
 * "INT4, FP8 and BF16": built from exponent and mantissa, subnormals,
 * infinities and NaN kept). */
double oracle_bf16_to_double(uint16_t bits) {
  int sign = (bits >> 15) & 1;
  int expo = (bits >> 7) & 0xFF;
  int mant = bits & 0x7F;
  double v;
  if (expo == 0xFF) {
    if (mant != 0) return NAN;
    v = INFINITY;
  } else if (expo == 0) {
    v = ldexp((double)mant / 128.0, -126);
  } else {
    v = ldexp(1.0 + (double)mant / 128.0, expo - 127);
  }
  return sign ? -v : v;
}

/* E4M3FN: sign, 4-bit exponent with bias 7, 3-bit mantissa; exponent 0 is
 * subnormal; S.1111.111 is NaN; there is no infinity ([glm-vx] checkpoint IO,
 * FP8 E4M3FN decoding). */
double oracle_e4m3fn_to_double(uint8_t bits) {
  int sign = (bits >> 7) & 1;
  int expo = (bits >> 3) & 0xF;
  int mant = bits & 0x7;
  double v;
  if (expo == 0xF && mant == 0x7) return NAN;
  if (expo == 0)
    v = ldexp((double)mant / 8.0, -6);
  else
    v = ldexp(1.0 + (double)mant / 8.0, expo - 7);
  return sign ? -v : v;
}

double oracle_f32_to_double(uint32_t bits) {
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static double decode_elem(const uint8_t *p, int dtype) {
  if (dtype == ORACLE_F32) {
    uint32_t b;
    memcpy(&b, p, 4);
    return oracle_f32_to_double(b);
  }
  if (dtype == ORACLE_BF16) {
    uint16_t b;
    memcpy(&b, p, 2);
    return oracle_bf16_to_double(b);
  }
  return oracle_e4m3fn_to_double(*p);
}

static int elem_bytes(int dtype) {
  return dtype == ORACLE_F32 ? 4 : (dtype == ORACLE_BF16 ? 2 : 1);
}

/* Decode a dense [count] vector stored in dtype. */
static void decode_vec(double *dst, const void *src, int64_t offset_elems, int count, int dtype) {
  const uint8_t *base = (const uint8_t *)src + offset_elems * elem_bytes(dtype);
  for (int i = 0; i < count; ++i) dst[i] = decode_elem(base + (int64_t)i * elem_bytes(dtype), dtype);
}

/* Decode token t of sequence seq from a cache into dst[width]; fp8 rows are
 * multiplied by the token's scale. */
static void load_row(double *dst, const oracle_cache *c, int32_t seq, int64_t t) {
  int64_t block = c->block_table ? (int64_t)c->block_table[(int64_t)seq * c->max_blocks + t / c->block_size]
                                 : (int64_t)seq;
  int64_t slot = t % c->block_size;
  const uint8_t *row = c->rows + block * c->block_stride + slot * c->row_stride;
  double s = 1.0;
  if (c->dtype == ORACLE_E4M3FN) s = (double)c->scale[block * c->scale_block_stride + slot];
  for (int d = 0; d < c->width; ++d) dst[d] = decode_elem(row + (int64_t)d * elem_bytes(c->dtype), c->dtype) * s;
}

/* ---------------------------------------------------------------- scores -- */

/* Lightning-indexer scores ([GLM-A100] "The model": every earlier token is
 * scored; "How do we know it is right?": ReLU per head, heads then combined).
 * q: [n_q][n_heads][keys->width] in q_dtype; w: [n_q][n_heads] float32.
 * Query i belongs to sequence q_seq[i] (q_seq may be NULL: all sequence 0) and
 * sees q_len[i] tokens.  scores[i * ld + s] is written for s < q_len[i] only. */
void oracle_index_scores(double *scores, int64_t ld, const void *q, int q_dtype, const float *w,
                         const oracle_cache *keys, const int32_t *q_seq, const int32_t *q_len, int32_t n_q,
                         int32_t n_heads) {
  const int D = keys->width;
  for (int32_t i = 0; i < n_q; ++i) {
    double *qi = (double *)malloc(sizeof(double) * (size_t)n_heads * D);
    decode_vec(qi, q, (int64_t)i * n_heads * D, n_heads * D, q_dtype);
    const int32_t seq = q_seq ? q_seq[i] : 0;
    const int64_t n = q_len[i];
#pragma omp parallel
    {
      double *k = (double *)malloc(sizeof(double) * D);
#pragma omp for schedule(static)
      for (int64_t s = 0; s < n; ++s) {
        load_row(k, keys, seq, s);
        double score = 0.0;
        for (int h = 0; h < n_heads; ++h) {
          double dot = 0.0;
          for (int d = 0; d < D; ++d) dot += qi[h * D + d] * k[d];
          double relu = dot > 0.0 ? dot : 0.0;
          score += (double)w[(int64_t)i * n_heads + h] * relu;
        }
        scores[i * ld + s] = score;
      }
      free(k);
    }
    free(qi);
  }
}

/* ------------------------------------------------------------------ top-k -- */

/* "a sorts strictly before b" for an ascending sort of the values -score, with
 * NaN after every number (numpy's placement). */
static int key_less(double a, double b) {
  if (isnan(a)) return 0;
  if (isnan(b)) return 1;
  return a < b;
}

/* Stable bottom-up merge sort of idx[0..n) by key[idx]: equal keys keep their
 * input order, which is what a stable argsort does. */
static void stable_argsort(int32_t *idx, int32_t *tmp, const double *key, int64_t n) {
  for (int64_t width = 1; width < n; width *= 2) {
    for (int64_t lo = 0; lo < n; lo += 2 * width) {
      int64_t mid = lo + width < n ? lo + width : n;
      int64_t hi = lo + 2 * width < n ? lo + 2 * width : n;
      int64_t a = lo, b = mid, o = lo;
      while (a < mid && b < hi) {
        /* take from the right run only if it is strictly smaller: stability */
        if (key_less(key[idx[b]], key[idx[a]]))
          tmp[o++] = idx[b++];
        else
          tmp[o++] = idx[a++];
      }
      while (a < mid) tmp[o++] = idx[a++];
      while (b < hi) tmp[o++] = idx[b++];
    }
    memcpy(idx, tmp, sizeof(int32_t) * (size_t)n);
  }
}

static int cmp_int32(const void *a, const void *b) {
  int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
  return (x > y) - (x < y);
}

/* Exact top-k ([GLM-A100] "The model": the k best, everything when fewer than k
 * tokens; "How do we know it is right?": the tie rule is a stable argsort of
 * -scores).  scores: [n_q][ld]; query i considers s < q_len[i].
 * indices: [n_q][k]; counts (nullable): [n_q] = min(k, q_len[i]).
 * order 0: kept indices ascending; order 1: argsort order. */
void oracle_topk(int32_t *indices, int32_t *counts, const double *scores, int64_t ld, const int32_t *q_len,
                 int32_t n_q, int32_t k, int order) {
#pragma omp parallel for schedule(dynamic)
  for (int32_t i = 0; i < n_q; ++i) {
    const int64_t n = q_len[i];
    double *neg = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    int32_t *tmp = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    for (int64_t s = 0; s < n; ++s) {
      neg[s] = -scores[i * ld + s];
      idx[s] = (int32_t)s;
    }
    stable_argsort(idx, tmp, neg, n);
    const int64_t kept = n < k ? n : k;
    int32_t *out = indices + (int64_t)i * k;
    for (int64_t j = 0; j < kept; ++j) out[j] = idx[j];
    if (order == 0) qsort(out, (size_t)kept, sizeof(int32_t), cmp_int32);
    for (int64_t j = kept; j < k; ++j) out[j] = -1;
    if (counts) counts[i] = (int32_t)kept;
    free(neg);
    free(idx);
    free(tmp);
  }
}

/* -------------------------------------------------------------- attention -- */

/* Softmax attention of one (query, head) over a list of latent rows, in the
 * absorbed-MLA form: logits z_j = scale * <q, row_j> over the full row,
 * weights softmax(z), output sum_j p_j * row_j[0:kv_lora].  Stable softmax:
 * the maximum is subtracted before exponentiation ([glm-vx] kernel list). */
static void attend_rows(double *out, double *lse, double *probs, const double *qh, const double *rows, int64_t m_rows,
                        int width, int kv_lora, double scale) {
  if (m_rows == 0) {
    for (int c = 0; c < kv_lora; ++c) out[c] = 0.0;
    *lse = -INFINITY;
    return;
  }
  double *z = (double *)malloc(sizeof(double) * (size_t)m_rows);
  double zmax = -INFINITY;
  for (int64_t j = 0; j < m_rows; ++j) {
    double dot = 0.0;
    for (int c = 0; c < width; ++c) dot += qh[c] * rows[j * width + c];
    z[j] = scale * dot;
    if (z[j] > zmax) zmax = z[j];
  }
  double l = 0.0;
  for (int64_t j = 0; j < m_rows; ++j) {
    z[j] = exp(z[j] - zmax);
    l += z[j];
  }
  for (int c = 0; c < kv_lora; ++c) {
    double acc = 0.0;
    for (int64_t j = 0; j < m_rows; ++j) acc += z[j] * rows[j * width + c];
    out[c] = acc / l;
  }
  if (probs)
    for (int64_t j = 0; j < m_rows; ++j) probs[j] = z[j] / l;
  *lse = zmax + log(l);
  free(z);
}

/* Sparse absorbed-MLA attention over the kept rows ([GLM-A100] "The model":
 * each query attends only to its kept tokens' latent vectors; [glm-vx]
 * absorbed MLA decode).  q: [n_q][n_heads][latent->width] in q_dtype;
 * indices: [n_q][k], entries < 0 skipped; out: [n_q][n_heads][kv_lora];
 * lse: [n_q][n_heads]; probs (nullable): [n_q][n_heads][k] softmax weight of
 * each index slot (0 for skipped slots). */
void oracle_mla_attend(double *out, double *lse, double *probs, const void *q, int q_dtype,
                       const oracle_cache *latent, int32_t kv_lora, const int32_t *indices, int32_t k,
                       const int32_t *q_seq, int32_t n_q, int32_t n_heads, double softmax_scale) {
  const int W = latent->width;
  double *rows = (double *)malloc(sizeof(double) * (size_t)k * W);
  int32_t *slot = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
  for (int32_t i = 0; i < n_q; ++i) {
    const int32_t seq = q_seq ? q_seq[i] : 0;
    int64_t m_rows = 0;
    for (int32_t j = 0; j < k; ++j) {
      int32_t t = indices[(int64_t)i * k + j];
      if (t < 0) continue;
      load_row(rows + m_rows * W, latent, seq, t);
      slot[m_rows++] = j;
    }
#pragma omp parallel for schedule(static)
    for (int32_t h = 0; h < n_heads; ++h) {
      double *qh = (double *)malloc(sizeof(double) * W);
      double *p = (double *)malloc(sizeof(double) * (size_t)k);
      decode_vec(qh, q, ((int64_t)i * n_heads + h) * W, W, q_dtype);
      attend_rows(out + ((int64_t)i * n_heads + h) * kv_lora, lse + (int64_t)i * n_heads + h, p, qh, rows, m_rows,
                  W, kv_lora, softmax_scale);
      if (probs) {
        double *pr = probs + ((int64_t)i * n_heads + h) * k;
        for (int32_t j = 0; j < k; ++j) pr[j] = 0.0;
        for (int64_t r = 0; r < m_rows; ++r) pr[slot[r]] = p[r];
      }
      free(qh);
      free(p);
    }
  }
  free(rows);
  free(slot);
}

/* Dense absorbed-MLA attention of each query over all its visible tokens
 * 0..q_len[i]-1.  Written directly as the textbook definition (no index list),
 * so that "sparse with k >= n equals dense" compares two separate codes. */
void oracle_mla_dense(double *out, double *lse, const void *q, int q_dtype, const oracle_cache *latent,
                      int32_t kv_lora, const int32_t *q_seq, const int32_t *q_len, int32_t n_q, int32_t n_heads,
                      double softmax_scale) {
  const int W = latent->width;
  for (int32_t i = 0; i < n_q; ++i) {
    const int32_t seq = q_seq ? q_seq[i] : 0;
    const int64_t n = q_len[i];
    double *row = (double *)malloc(sizeof(double) * W);
    double *qh = (double *)malloc(sizeof(double) * W);
    double *z = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (int32_t h = 0; h < n_heads; ++h) {
      double *o = out + ((int64_t)i * n_heads + h) * kv_lora;
      decode_vec(qh, q, ((int64_t)i * n_heads + h) * W, W, q_dtype);
      if (n == 0) {
        for (int c = 0; c < kv_lora; ++c) o[c] = 0.0;
        lse[(int64_t)i * n_heads + h] = -INFINITY;
        continue;
      }
      double zmax = -INFINITY;
      for (int64_t t = 0; t < n; ++t) {
        load_row(row, latent, seq, t);
        double dot = 0.0;
        for (int c = 0; c < W; ++c) dot += qh[c] * row[c];
        z[t] = softmax_scale * dot;
        if (z[t] > zmax) zmax = z[t];
      }
      double l = 0.0;
      for (int c = 0; c < kv_lora; ++c) o[c] = 0.0;
      for (int64_t t = 0; t < n; ++t) {
        double p = exp(z[t] - zmax);
        l += p;
        load_row(row, latent, seq, t);
        for (int c = 0; c < kv_lora; ++c) o[c] += p * row[c];
      }
      for (int c = 0; c < kv_lora; ++c) o[c] /= l;
      lse[(int64_t)i * n_heads + h] = zmax + log(l);
    }
    free(row);
    free(qh);
    free(z);
  }
}

/* ------------------------------------------------------------ decode step -- */

/* One DSA decode step for `batch` sequences: sequence b has seq_len[b] tokens
 * and its query (the newest token) sees all of them.  Scores, then top-k
 * (ascending index order), then sparse attention.  scores_out: [batch][ld]
 * (required: the top-k reads it); indices_out: [batch][k]. */
void oracle_decode_step(double *out, double *lse, double *scores_out, int64_t ld, int32_t *indices_out,
                        const void *q_idx, int q_idx_dtype, const float *w_idx, const oracle_cache *keys,
                        int32_t idx_heads, const void *q_mla, int q_mla_dtype, const oracle_cache *latent,
                        int32_t kv_lora, int32_t mla_heads, const int32_t *seq_len, int32_t batch, int32_t k,
                        double softmax_scale) {
  int32_t *seq = (int32_t *)malloc(sizeof(int32_t) * (size_t)(batch > 0 ? batch : 1));
  for (int32_t b = 0; b < batch; ++b) seq[b] = b;
  oracle_index_scores(scores_out, ld, q_idx, q_idx_dtype, w_idx, keys, seq, seq_len, batch, idx_heads);
  oracle_topk(indices_out, NULL, scores_out, ld, seq_len, batch, k, 0);
  oracle_mla_attend(out, lse, NULL, q_mla, q_mla_dtype, latent, kv_lora, indices_out, k, seq, batch, mla_heads,
                    softmax_scale);
  free(seq);
}

/* ------------------------------------------------------ absorption GEMMs -- */

/* Query absorption of absorbed MLA ([glm-vx] component list: absorbed MLA
 * decode; [GLM-A100] "The model": keys and values are kept as one compressed
 * latent row per token).  The key a head would see is the up-projection of
 * the latent row, k_h = W_UK[h]^T latent[0..kv_lora); absorbing W_UK into the
 * query gives the same logit from the latent row directly:
 *     q_out[i][h][c] = sum_d q_nope[i][h][d] * w_uk[h][d][c],   c < kv_lora
 *     q_out[i][h][kv_lora + r] = q_rope[i][h][r],              r < rope
 * (the rope part of the row is compared against the query's rope part as is).
 * q_nope [n_q][H][d_nope] and q_rope [n_q][H][rope] (may be NULL when rope =
 * 0) in q_dtype; w_uk [H][d_nope][kv_lora] bf16; q_out [n_q][H][kv_lora + rope]
 * double. */
void oracle_mla_absorb_q(double *q_out, const void *q_nope, const void *q_rope, int q_dtype, const uint16_t *w_uk,
                         int32_t n_q, int32_t H, int32_t d_nope, int32_t kv_lora, int32_t rope) {
  const int W = kv_lora + rope;
  for (int32_t i = 0; i < n_q; ++i) {
    for (int32_t h = 0; h < H; ++h) {
      double *dst = q_out + ((int64_t)i * H + h) * W;
      for (int c = 0; c < kv_lora; ++c) {
        double acc = 0.0;
        for (int d = 0; d < d_nope; ++d) {
          const double qv = decode_elem((const uint8_t *)q_nope + (((int64_t)i * H + h) * d_nope + d) * elem_bytes(q_dtype),
                                        q_dtype);
          acc += qv * oracle_bf16_to_double(w_uk[((int64_t)h * d_nope + d) * kv_lora + c]);
        }
        dst[c] = acc;
      }
      for (int r = 0; r < rope; ++r)
        dst[kv_lora + r] = decode_elem((const uint8_t *)q_rope + (((int64_t)i * H + h) * rope + r) * elem_bytes(q_dtype),
                                       q_dtype);
    }
  }
}

/* Output up-projection of absorbed MLA: the attention over latent rows gives
 * o_lat[i][h] = sum_j p_j latent_j[0..kv_lora), and the head's output in value
 * space is its projection by W_UV (the value of row j is W_UV[h]^T latent_j, so
 * the projection of the weighted sum equals the weighted sum of the values):
 *     out[i][h][e] = sum_c o_lat[i][h][c] * w_uv[h][c][e],   e < d_v
 * o_lat [n_q][H][kv_lora] float32; w_uv [H][kv_lora][d_v] bf16; out double. */
void oracle_mla_absorb_out(double *out, const float *o_lat, const uint16_t *w_uv, int32_t n_q, int32_t H,
                           int32_t kv_lora, int32_t d_v) {
  for (int32_t i = 0; i < n_q; ++i) {
    for (int32_t h = 0; h < H; ++h) {
      const float *src = o_lat + ((int64_t)i * H + h) * kv_lora;
      double *dst = out + ((int64_t)i * H + h) * d_v;
      for (int e = 0; e < d_v; ++e) {
        double acc = 0.0;
        for (int c = 0; c < kv_lora; ++c)
          acc += (double)src[c] * oracle_bf16_to_double(w_uv[((int64_t)h * kv_lora + c) * d_v + e]);
        dst[e] = acc;
      }
    }
  }
}

/* ----------------------------------------------------------- cache append -- */

/* e4m3fn encoding of a float32 value, for writing keys into an fp8 cache
 * ([GLM-A100] "INT4, FP8 and BF16": FP8 is E4M3 bytes with a float32 scale;
 * [glm-vx] component list: E4M3FN).  The pages only decode; the reading taken
 * for encoding is round to nearest with ties to the even code, magnitudes at or
 * above the largest finite value (448) saturated to it, and the sign bit of x
 * kept (negative values that round to zero give 0x80).  The code is found by a
 * plain search: the largest non-negative finite code whose decoded value does
 * not exceed |x|, then a comparison with the midpoint to the next code (the
 * midpoint of two neighbouring e4m3fn values is exact in double).  Finite
 * inputs only. */
uint8_t oracle_e4m3fn_quantize(float x) {
  uint32_t bits;
  memcpy(&bits, &x, sizeof bits);
  const uint8_t sign = (uint8_t)((bits >> 31) << 7);
  const double m = fabs((double)x);
  if (m >= 448.0) return (uint8_t)(sign | 0x7E);
  int lo = 0;
  for (int c = 1; c <= 0x7E; ++c)
    if (oracle_e4m3fn_to_double((uint8_t)c) <= m) lo = c;
  const double mid = 0.5 * (oracle_e4m3fn_to_double((uint8_t)lo) + oracle_e4m3fn_to_double((uint8_t)(lo + 1)));
  int c = lo;
  if (m > mid || (m == mid && (lo & 1))) c = lo + 1;
  return (uint8_t)(sign | c);
}

/* Per-token scale of an fp8 key row (reading: the pages give E4M3 with float32
 * scales but no rule for choosing them).  The row's largest magnitude maps to
 * the largest finite code: s = amax / 448, floored at the smallest normal
 * float (2^-126) so an all-zero row gets a usable positive scale.  Computed in
 * float32, the precision the encoded byte is decided in. */
float oracle_key_scale(const float *k, int n) {
  float amax = 0.0f;
  for (int d = 0; d < n; ++d) {
    const float a = fabsf(k[d]);
    if (a > amax) amax = a;
  }
  float s = amax / 448.0f;
  const float floor_s = 0x1p-126f;
  return s < floor_s ? floor_s : s;
}

static float input_to_float(const void *src, int64_t i, int dtype) {
  if (dtype == ORACLE_BF16) {
    uint16_t b;
    memcpy(&b, (const uint8_t *)src + i * 2, 2);
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
  }
  float f;
  memcpy(&f, (const uint8_t *)src + i * 4, 4);
  return f;
}

/* Token i's row into one cache: fp8 caches get s = oracle_key_scale(row) and
 * byte d = oracle_e4m3fn_quantize(x[d] / s) (float32 division) with scale s;
 * other caches get the input bits copied (the input is in the cache's dtype). */
static void append_row(const oracle_cache *c, const void *src, int src_dtype, int32_t i, int32_t b, int64_t t) {
  const int W = c->width;
  const int64_t block = c->block_table ? (int64_t)c->block_table[(int64_t)b * c->max_blocks + t / c->block_size]
                                       : (int64_t)b;
  const int64_t slot = t % c->block_size;
  uint8_t *row = (uint8_t *)c->rows + block * c->block_stride + slot * c->row_stride;
  if (c->dtype == ORACLE_E4M3FN) {
    float *x = (float *)calloc((size_t)(W > 0 ? W : 1), sizeof(float));
    for (int d = 0; d < W; ++d) x[d] = input_to_float(src, (int64_t)i * W + d, src_dtype);
    const float s = oracle_key_scale(x, W);
    for (int d = 0; d < W; ++d) row[d] = oracle_e4m3fn_quantize(x[d] / s);
    ((float *)c->scale)[block * c->scale_block_stride + slot] = s;
    free(x);
  } else {
    const int eb = elem_bytes(c->dtype);
    memcpy(row, (const uint8_t *)src + (int64_t)i * W * eb, (size_t)W * eb);
  }
}

/* Write new tokens into the caches (the step before the path: a token's key
 * and latent row must be in place before a query sees it, [GLM-A100] "The
 * model": every earlier token is scored, the query's own included).  Token i
 * (sequence seq ? seq[i] : 0, position pos[i]) goes to both caches (either may
 * be NULL) through append_row: fp8 caches, keys or latent rows, are quantized
 * with the row's own float32 scale; others are copied.
 * new_keys: [n_new][keys->width] in new_keys_dtype; new_latent: [n_new]
 * [latent->width] in new_latent_dtype (f32 or bf16). */
void oracle_cache_append(const oracle_cache *keys, const void *new_keys, int new_keys_dtype,
                         const oracle_cache *latent, const void *new_latent, int new_latent_dtype,
                         const int32_t *seq, const int32_t *pos, int32_t n_new) {
  for (int32_t i = 0; i < n_new; ++i) {
    const int32_t b = seq ? seq[i] : 0;
    const int64_t t = pos[i];
    if (keys) append_row(keys, new_keys, new_keys_dtype, i, b, t);
    if (latent) append_row(latent, new_latent, new_latent_dtype, i, b, t);
  }
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads for the oracle's later parallel loops (timing only; results do not
   depend on it). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
