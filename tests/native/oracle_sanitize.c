/* Memory and undefined-behaviour check of the CPU oracle (test infrastructure).
 * Built together with oracle/dsa_oracle.c under AddressSanitizer and
 * UndefinedBehaviorSanitizer by tests/test_sanitizers.py, it calls every oracle
 * entry point on small seeded inputs: contiguous and paged caches, f32, bf16
 * and fp8 rows, top-k in both orders with n < k, n = 0, NaN and ties,
 * attention with empty slots.  Values are not checked here (the Python pins
 * do that); the sanitizers abort on any invalid access or undefined operation.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

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

double oracle_bf16_to_double(uint16_t bits);
double oracle_e4m3fn_to_double(uint8_t bits);
void oracle_index_scores(double *scores, int64_t ld, const void *q, int q_dtype, const float *w,
                         const oracle_cache *keys, const int32_t *q_seq, const int32_t *q_len, int32_t n_q,
                         int32_t n_heads);
void oracle_topk(int32_t *indices, int32_t *counts, const double *scores, int64_t ld, const int32_t *q_len,
                 int32_t n_q, int32_t k, int order);
void oracle_mla_attend(double *out, double *lse, double *probs, const void *q, int q_dtype,
                       const oracle_cache *latent, int32_t kv_lora, const int32_t *indices, int32_t k,
                       const int32_t *q_seq, int32_t n_q, int32_t n_heads, double softmax_scale);
void oracle_mla_dense(double *out, double *lse, const void *q, int q_dtype, const oracle_cache *latent,
                      int32_t kv_lora, const int32_t *q_seq, const int32_t *q_len, int32_t n_q, int32_t n_heads,
                      double softmax_scale);
void oracle_decode_step(double *out, double *lse, double *scores_out, int64_t ld, int32_t *indices_out,
                        const void *q_idx, int q_idx_dtype, const float *w_idx, const oracle_cache *keys,
                        int32_t idx_heads, const void *q_mla, int q_mla_dtype, const oracle_cache *latent,
                        int32_t kv_lora, int32_t mla_heads, const int32_t *seq_len, int32_t batch, int32_t k,
                        double softmax_scale);
void oracle_mla_absorb_q(double *q_out, const void *q_nope, const void *q_rope, int q_dtype, const uint16_t *w_uk,
                         int32_t n_q, int32_t H, int32_t d_nope, int32_t kv_lora, int32_t rope);
void oracle_mla_absorb_out(double *out, const float *o_lat, const uint16_t *w_uv, int32_t n_q, int32_t H,
                           int32_t kv_lora, int32_t d_v);
uint8_t oracle_e4m3fn_quantize(float x);
float oracle_key_scale(const float *k, int n);
void oracle_cache_append(const oracle_cache *keys, const void *new_keys, int new_keys_dtype,
                         const oracle_cache *latent, const void *new_latent, int new_latent_dtype,
                         const int32_t *seq, const int32_t *pos, int32_t n_new);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {
  state = state * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(state >> 32);
}
static float next_normalish(void) { return ((float)(next_u32() >> 8) / 16777216.0f - 0.5f) * 4.0f; }

static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

/* rows of `dtype` (0 f32, 1 bf16, 2 fp8) for `nseq` sequences of `cap` tokens,
 * contiguous or paged in blocks of 64 with a shuffled table */
typedef struct {
  oracle_cache c;
  uint8_t *rows;
  float *scale;
  int32_t *table;
} cache_buf;

static cache_buf make_cache(int dtype, int width, int nseq, int cap, int paged) {
  cache_buf b;
  memset(&b, 0, sizeof b);
  const int eb = dtype == 0 ? 4 : (dtype == 1 ? 2 : 1);
  const int bs = paged ? 64 : cap;
  const int per = (cap + bs - 1) / bs;
  const int nblocks = paged ? nseq * per : nseq;
  b.rows = (uint8_t *)malloc((size_t)nblocks * bs * width * eb);
  for (size_t i = 0; i < (size_t)nblocks * bs * width; ++i) {
    const float v = next_normalish();
    if (dtype == 0) memcpy(b.rows + 4 * i, &v, 4);
    else if (dtype == 1) { uint16_t h = to_bf16(v); memcpy(b.rows + 2 * i, &h, 2); }
    else b.rows[i] = oracle_e4m3fn_quantize(v);
  }
  if (dtype == 2) {
    b.scale = (float *)malloc(sizeof(float) * (size_t)nblocks * bs);
    for (int i = 0; i < nblocks * bs; ++i) b.scale[i] = 0.5f + (float)(next_u32() % 1000) / 666.0f;
  }
  if (paged) {
    b.table = (int32_t *)malloc(sizeof(int32_t) * (size_t)nseq * per);
    for (int i = 0; i < nseq * per; ++i) b.table[i] = i;
    for (int i = nseq * per - 1; i > 0; --i) {
      const int j = (int)(next_u32() % (uint32_t)(i + 1));
      const int32_t t = b.table[i];
      b.table[i] = b.table[j];
      b.table[j] = t;
    }
  }
  b.c.rows = b.rows;
  b.c.scale = b.scale;
  b.c.row_stride = (int64_t)width * eb;
  b.c.block_stride = (int64_t)bs * width * eb;
  b.c.scale_block_stride = bs;
  b.c.block_table = b.table;
  b.c.block_size = bs;
  b.c.max_blocks = paged ? per : 0;
  b.c.width = width;
  b.c.dtype = dtype;
  return b;
}

static void free_cache(cache_buf *b) {
  free(b->rows);
  free(b->scale);
  free(b->table);
}

static void *make_q(int dtype, size_t n) {
  if (dtype == 0) {
    float *q = (float *)malloc(4 * n);
    for (size_t i = 0; i < n; ++i) q[i] = next_normalish();
    return q;
  }
  uint16_t *q = (uint16_t *)malloc(2 * n);
  for (size_t i = 0; i < n; ++i) q[i] = to_bf16(next_normalish());
  return q;
}

static double checksum = 0.0;
static void take(const double *x, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (isfinite(x[i])) checksum += x[i];
}

static void run_config(int key_dt, int lat_dt, int paged, int D, int Hi, int W, int L, int H, int k) {
  const int B = 3, cap = 300;
  const int32_t lens[3] = {0, 77, 300};
  cache_buf keys = make_cache(key_dt, D, B, cap, paged);
  cache_buf lat = make_cache(lat_dt, W, B, cap, paged);
  const int qk_dt = key_dt == 0 ? 0 : 1, qm_dt = lat_dt == 0 ? 0 : 1;
  void *q_idx = make_q(qk_dt, (size_t)B * Hi * D);
  void *q_mla = make_q(qm_dt, (size_t)B * H * W);
  float *w = (float *)malloc(sizeof(float) * B * Hi);
  for (int i = 0; i < B * Hi; ++i) w[i] = next_normalish();
  const int64_t ld = cap + 5;
  double *scores = (double *)malloc(sizeof(double) * B * ld);
  for (int64_t i = 0; i < B * ld; ++i) scores[i] = NAN;
  int32_t seq[3] = {0, 1, 2};
  oracle_index_scores(scores, ld, q_idx, qk_dt, w, &keys.c, seq, lens, B, Hi);
  scores[2 * ld + 10] = NAN;                      /* special values and ties for the top-k */
  scores[2 * ld + 11] = -0.0;
  scores[2 * ld + 12] = 0.0;
  scores[2 * ld + 13] = scores[2 * ld + 14];
  int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * B * k);
  int32_t cnt[3];
  for (int order = 0; order < 2; ++order) oracle_topk(idx, cnt, scores, ld, lens, B, k, order);
  double *out = (double *)malloc(sizeof(double) * B * H * L);
  double *lse = (double *)malloc(sizeof(double) * B * H);
  double *probs = (double *)malloc(sizeof(double) * B * H * k);
  idx[k + 1] = -1;                                /* an empty slot inside a row */
  oracle_mla_attend(out, lse, probs, q_mla, qm_dt, &lat.c, L, idx, k, seq, B, H, 0.05);
  take(out, (size_t)B * H * L);
  oracle_mla_dense(out, lse, q_mla, qm_dt, &lat.c, L, seq, lens, B, H, 0.05);
  take(out, (size_t)B * H * L);
  oracle_decode_step(out, lse, scores, ld, idx, q_idx, qk_dt, w, &keys.c, Hi, q_mla, qm_dt, &lat.c, L, H, lens, B, k,
                     0.05);
  take(out, (size_t)B * H * L);
  take(scores, (size_t)B * ld);
  /* append two tokens to both caches (keys quantized when fp8) */
  const int32_t aseq[2] = {1, 2}, apos[2] = {77, 299};
  if (key_dt != 0) {
    uint16_t *nk = (uint16_t *)make_q(1, 2 * (size_t)D);
    void *nl = make_q(lat_dt == 0 ? 0 : 1, 2 * (size_t)W);
    oracle_cache_append(&keys.c, nk, 1, &lat.c, nl, lat_dt == 0 ? 0 : 1, aseq, apos, 2);
    free(nk);
    free(nl);
  } else {
    float *nk = (float *)make_q(0, 2 * (size_t)D);
    float *nl = (float *)make_q(0, 2 * (size_t)W);
    oracle_cache_append(&keys.c, nk, 0, &lat.c, nl, 0, aseq, apos, 2);
    free(nk);
    free(nl);
  }
  free(q_idx);
  free(q_mla);
  free(w);
  free(scores);
  free(idx);
  free(out);
  free(lse);
  free(probs);
  free_cache(&keys);
  free_cache(&lat);
}

int main(void) {
  for (int c = 0; c < 65536; ++c) checksum += isfinite(oracle_bf16_to_double((uint16_t)c)) ? 1.0 : 0.0;
  for (int c = 0; c < 256; ++c) checksum += isfinite(oracle_e4m3fn_to_double((uint8_t)c)) ? 1.0 : 0.0;
  const float specials[] = {0.0f, -0.0f, 1e-30f, 448.0f, 500.0f, -1e6f, 0.0009765625f, 3.0e-3f};
  for (size_t i = 0; i < sizeof specials / sizeof specials[0]; ++i) checksum += oracle_e4m3fn_quantize(specials[i]);
  float row[5] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  checksum += oracle_key_scale(row, 5);
  run_config(0, 0, 0, 32, 4, 80, 64, 8, 64);     /* fp32, contiguous */
  run_config(1, 1, 1, 128, 32, 576, 512, 16, 100);  /* bf16, paged */
  run_config(2, 1, 0, 128, 5, 576, 512, 16, 300);   /* fp8 keys, k = capacity */
  run_config(2, 2, 1, 64, 7, 576, 512, 16, 33);     /* fp8 keys and fp8 latent rows, paged */
  {
    const int nq = 2, Hh = 3, dn = 32, kl = 64, r = 16, dv = 64;
    uint16_t *qn = (uint16_t *)make_q(1, (size_t)nq * Hh * dn), *qr = (uint16_t *)make_q(1, (size_t)nq * Hh * r);
    uint16_t *wuk = (uint16_t *)make_q(1, (size_t)Hh * dn * kl), *wuv = (uint16_t *)make_q(1, (size_t)Hh * kl * dv);
    float *ol = (float *)make_q(0, (size_t)nq * Hh * kl);
    double *o1 = (double *)malloc(sizeof(double) * nq * Hh * (kl + r)), *o2 = (double *)malloc(sizeof(double) * nq * Hh * dv);
    oracle_mla_absorb_q(o1, qn, qr, 1, wuk, nq, Hh, dn, kl, r);
    oracle_mla_absorb_q(o1, qn, NULL, 1, wuk, nq, Hh, dn, kl, 0);
    oracle_mla_absorb_out(o2, ol, wuv, nq, Hh, kl, dv);
    take(o1, (size_t)nq * Hh * kl);
    take(o2, (size_t)nq * Hh * dv);
    free(qn); free(qr); free(wuk); free(wuv); free(ol); free(o1); free(o2);
  }
  printf("oracle sanitizer run ok (checksum %.6g)\n", checksum);
  return 0;
}
