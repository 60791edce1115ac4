/*
 * dsa.h -- C ABI of libdsa, the MI355X (gfx950) DeepSeek-style sparse attention
 * (DSA) hot path of the GLM-5 decoder:
 *
 *   1. a lightning indexer scores every earlier token of each query,
 *   2. an exact top-k keeps the best k tokens (all of them below k tokens),
 *   3. absorbed MLA attention runs over the compressed latent rows of only the
 *      kept tokens.
 *
 * The operations are the ones the page "GLM on an A100, in Vx" defines in its
 * section "The model" (latent K/V per token, an indexer that scores every
 * earlier token, the best 2,048 kept, everything kept below 2,048 tokens) and in
 * "How do we know it is right?" (ReLU per indexer head before the heads are
 * combined; ties broken as a stable argsort of -scores).  The page
 * "Self-contained GLM-5 serving stack" names the pieces (absorbed MLA decode,
 * compressed request-local KV, full DSA indexer selection, fused GPU index-score
 * kernel, split online-softmax compressed MLA).
 *
 * Conventions for every entry point:
 *   - All array arguments are DEVICE pointers to caller-owned memory, except the
 *     dsa_cache descriptor structs themselves, which live in host memory and
 *     are read during the call only.  The library allocates nothing, frees
 *     nothing and keeps no state between calls.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream) and
 *     the call returns after enqueue: no host<->device copies, no device reads
 *     on the host, no synchronization.  Producers on other streams must be
 *     ordered before the call by the caller (events).
 *   - Arguments are validated on the host before any HIP call.  Sizes of 0 queries
 *     return DSA_OK with no work.  Negative sizes, NULL required pointers, k < 1
 *     or inconsistent strides return DSA_ERR_INVALID_ARGUMENT; shapes or dtypes
 *     outside the supported set return DSA_ERR_UNSUPPORTED (there is no fallback
 *     path); a workspace smaller than the matching *_workspace_size() returns
 *     DSA_ERR_WORKSPACE_TOO_SMALL; a failed launch returns DSA_ERR_DEVICE.
 *   - Values that live on the device (lengths, block tables, indices) are
 *     trusted: an out-of-range value is undefined behaviour.
 *   - Workspaces must be zero-filled before their first use (for example with
 *     dsa_workspace_clear) and are left zero-filled in their control words by every
 *     call, so one workspace can serve any number of consecutive calls on one
 *     stream.  Calls that share a workspace must not overlap in time.
 *   - Results are deterministic: the same inputs give the same bits on every run.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARGUMENT = 1,
  DSA_ERR_UNSUPPORTED = 2,
  DSA_ERR_WORKSPACE_TOO_SMALL = 3,
  DSA_ERR_DEVICE = 4
} dsa_status;

typedef enum {
  DSA_F32 = 0,        /* IEEE binary32 */
  DSA_BF16 = 1,       /* bfloat16, raw 16-bit patterns */
  DSA_FP8_E4M3FN = 2  /* OCP float8 e4m3fn bytes (bias 7, no infinity, 0x7F/0xFF NaN) */
} dsa_dtype;

/*
 * A per-token row cache in device memory ("compressed request-local KV").
 * Token t of sequence b is stored at
 *     rows + p * block_stride + (t % block_size) * row_stride          (bytes)
 * where p = block_table ? block_table[b * max_blocks + t / block_size] : b.
 *   - Contiguous caches: block_table = NULL and block_size = the capacity (rows
 *     per sequence); p is then the sequence index.
 *   - Paged caches: block_table is an int32 device array [batch][max_blocks]
 *     and block_size a multiple of 32 (64 in the GLM-5 layout).  The key and
 *     latent caches may share one table.
 *   - fp8 rows carry one float32 scale per token (the dequantized value is
 *     e4m3fn(byte) * scale), at scale[p * scale_block_stride + t % block_size];
 *     scale is ignored for other dtypes.
 *   - rows, row_stride and block_stride must be multiples of 16 bytes, and
 *     row_stride >= width * element size.  A row_stride above 16 MiB returns
 *     DSA_ERR_UNSUPPORTED.
 *   - The row at `rows` itself (and, when paged, entry 0 of every addressed
 *     sequence's block table row) must be readable whenever a call has work:
 *     -1 index slots load it in place of a token and discard the value.
 */
typedef struct {
  const void *rows;
  const float *scale;
  int64_t row_stride;          /* bytes between consecutive tokens of a block */
  int64_t block_stride;        /* bytes between blocks (or sequences) */
  int64_t scale_block_stride;  /* floats between blocks of scales (fp8 only) */
  const int32_t *block_table;  /* NULL: contiguous */
  int32_t block_size;          /* tokens per block; contiguous: capacity */
  int32_t max_blocks;          /* row length of block_table (paged only) */
  int32_t width;               /* elements per row */
  dsa_dtype dtype;
} dsa_cache;

/* dsa_topk flags: the order in which a row's kept indices are written */
#define DSA_TOPK_ORDER_INDEX 0u  /* ascending token order (the default) */
#define DSA_TOPK_ORDER_SCORE 1u  /* the stable argsort order of -scores ("GLM on an A100, in Vx", "How do we know
                                    it is right?"): score descending, equal scores by ascending token index */

/*
 * Lightning-indexer scores.  For query i of sequence seq = q_seq ? q_seq[i] : 0
 * that sees n = q_len[i] tokens (its own included), for every token s < n:
 *     scores[i * ld_scores + s] = sum_h w[i * n_heads + h] * max(0, sum_d q[i][h][d] * khat[s][d])
 * with khat = the key row (fp8: e4m3fn(byte) * scale[s]).  One key row of
 * width keys->width is shared by all indexer heads.  Entries s >= n are not
 * written.  Accumulation is float32.
 *   q       [n_q][n_heads][keys->width], dtype q_dtype
 *   w       [n_q][n_heads] float32 (any sign)
 *   q_len   [n_q] int32, 0 <= q_len[i] <= max_len (device)
 *   q_seq   [n_q] int32 or NULL (all queries in sequence 0)
 * Supported: q f32 with f32 keys, or q bf16 with bf16 or fp8 keys;
 *   width 32..128 in steps of 32 (bf16/fp8 keys: 64 or 128); 1 <= n_heads <= 64;
 *   ld_scores >= max_len; n_q <= 65535.
 */
dsa_status dsa_index_scores(float *scores, int64_t ld_scores, const void *q, dsa_dtype q_dtype, const float *w,
                            const dsa_cache *keys, const int32_t *q_seq, const int32_t *q_len, int32_t n_q,
                            int32_t n_heads, int32_t max_len, void *stream);

/*
 * Exact top-k.  For query i with n = q_len[i], keeps the first min(k, n)
 * entries of a stable descending sort of scores[i * ld_scores + s], s < n:
 * ties go to the lower token index, -0.0 equals +0.0, NaN ranks below every
 * number.  indices [n_q][k] int32 receive the kept token indices followed by
 * -1 padding, in ascending token order (flags = DSA_TOPK_ORDER_INDEX) or in the
 * stable argsort order of -scores (DSA_TOPK_ORDER_SCORE: score descending,
 * equal scores by ascending index; the same set, reordered by a sort of the
 * kept entries); counts [n_q] (nullable) receive min(k, n).  Selection and
 * ordering are integer-only on an order-preserving 32-bit image of each score,
 * so the result is exact and deterministic.  Other flags return
 * DSA_ERR_UNSUPPORTED.  Every row of scores must be readable up to max_len
 * floats (the kernels may read past a row's visible count, never past
 * max_len).
 * Supported: 1 <= k <= 2048, 1 <= max_len <= 262144, n_q <= 65535.
 */
dsa_status dsa_topk(int32_t *indices, int32_t *counts, const float *scores, int64_t ld_scores,
                    const int32_t *q_len, int32_t n_q, int32_t k, int32_t max_len, uint32_t flags,
                    void *workspace, size_t workspace_bytes, void *stream);
size_t dsa_topk_workspace_size(int32_t n_q, int32_t k, int32_t max_len);

/*
 * Sparse absorbed-MLA attention over kept latent rows.  For query i (sequence
 * q_seq ? q_seq[i] : 0) and head h, over the slots j with indices[i * k + j] >= 0:
 *     z_j = softmax_scale * sum_{c < W} q[i][h][c] * row_j[c]      (W = latent->width)
 *     out[i][h][c] = sum_j softmax(z)_j * row_j[c],  c < kv_lora
 *     lse[i][h]    = ln sum_j exp(z_j)
 * The key is the whole latent row (kv_lora latent + rope), the value its
 * first kv_lora entries.  No kept slot: out = 0, lse = -inf.
 *   q       [n_q][n_heads][W], dtype q_dtype (the latent dtype, or bf16 for an
 *           fp8 latent cache)
 *   out     [n_q][n_heads][kv_lora] float32;  lse [n_q][n_heads] float32 (nullable)
 * An fp8 latent cache holds e4m3fn rows with one float32 scale per token
 * (row_j = e4m3fn(bytes) * scale[token], the dsa_cache fp8 convention): the
 * memory-halving variant of the FP8 E4M3 + float32-scale format of "GLM on an
 * A100, in Vx", "INT4, FP8 and BF16"; dsa_cache_append writes it.
 * Supported: bf16 q with bf16 or fp8 latent rows, W = 576, kv_lora = 512,
 *   n_heads a multiple of 16 up to 128; f32 with W <= 1024 a multiple of 4,
 *   kv_lora <= W a multiple of 4, n_heads <= 128; 1 <= k <= 2048;
 *   n_q * n_heads < 2^24 (the launches stay below 2^32 work-items per grid
 *   dimension; DSA_ERR_UNSUPPORTED beyond).
 */
dsa_status mla_sparse_attend(float *out, float *lse, const void *q, dsa_dtype q_dtype, const dsa_cache *latent,
                             int32_t kv_lora, const int32_t *indices, int32_t k, const int32_t *q_seq, int32_t n_q,
                             int32_t n_heads, float softmax_scale, void *workspace, size_t workspace_bytes,
                             void *stream);
size_t mla_sparse_attend_workspace_size(int32_t n_q, int32_t n_heads, int32_t kv_lora, int32_t k);

/*
 * One fused DSA decode step for `batch` sequences: sequence b has seq_len[b]
 * tokens and its newest token's query sees all of them.  Runs the indexer
 * (scores), the exact top-k (ascending index order) and sparse MLA attention,
 * stream-ordered, with the same definitions as the three calls above.
 *   q_idx [batch][idx_heads][keys->width], w_idx [batch][idx_heads]
 *   q_mla [batch][mla_heads][latent->width]
 *   out [batch][mla_heads][kv_lora], lse [batch][mla_heads] (nullable)
 *   scores_out [batch][max_len] float32 and indices_out [batch][k] int32 are
 *   optional (NULL) copies of the intermediate scores and kept indices.
 * Supported: the union of the constraints of the three calls.
 */
dsa_status dsa_decode_step(float *out, float *lse, const void *q_idx, dsa_dtype q_idx_dtype, const float *w_idx,
                           const dsa_cache *keys, int32_t idx_heads, const void *q_mla, dsa_dtype q_mla_dtype,
                           const dsa_cache *latent, int32_t kv_lora, int32_t mla_heads, const int32_t *seq_len,
                           int32_t batch, int32_t max_len, int32_t k, float softmax_scale, float *scores_out,
                           int32_t *indices_out, void *workspace, size_t workspace_bytes, void *stream);
size_t dsa_decode_step_workspace_size(int32_t batch, int32_t max_len, int32_t k, int32_t mla_heads,
                                      int32_t kv_lora);

/*
 * dsa_decode_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments without the workspace, the same results bit for bit.
 * The step's scratch is a static device array of DSA_NOALLOC_SCRATCH_BYTES
 * inside the library, one per GPU, held until the process ends; the call
 * allocates and frees nothing.  A shape whose dsa_decode_step_workspace_size
 * exceeds that size returns DSA_ERR_WORKSPACE_TOO_SMALL (for example, 4 x
 * 131072 tokens needs about 14 MiB and 16 x 32768 about 38 MiB; 96 x 16384
 * (55 MiB) does not fit).  Every call on one GPU shares that GPU's array: calls that
 * overlap in time on one GPU (two streams, two host threads) race and must
 * be ordered by the caller.  The first call on a device looks up the array's
 * device address (hipGetSymbolAddress) with that device current.
 */
#define DSA_NOALLOC_SCRATCH_BYTES ((size_t)48 << 20)
dsa_status dsa_decode_step_noalloc(float *out, float *lse, const void *q_idx, dsa_dtype q_idx_dtype,
                                   const float *w_idx, const dsa_cache *keys, int32_t idx_heads, const void *q_mla,
                                   dsa_dtype q_mla_dtype, const dsa_cache *latent, int32_t kv_lora,
                                   int32_t mla_heads, const int32_t *seq_len, int32_t batch, int32_t max_len,
                                   int32_t k, float softmax_scale, float *scores_out, int32_t *indices_out,
                                   void *stream);

/*
 * One fused DSA decode step over a multi-token window ("GLM 5.3 Flash
 * (strata-poly)", section "How it uses the card", "Guessing ahead", and the
 * --window option: the known token and up to three guesses go through the
 * model together).  Sequence b holds seq_len[b] tokens, the last `window` of
 * them the window's tokens: query j (0 <= j < window) of sequence b is the
 * token at 0-based position seq_len[b] - window + j and sees the
 * seq_len[b] - window + j + 1 tokens up to and including itself (0 when that is
 * not positive: the query sees nothing, keeps no index, out = 0, lse = -inf).
 * Each query's result is that of a single-token step whose sequence ends at its
 * position: the same scores and indices; attention within the tolerance of
 * the split order.
 *   queries are row i = b * window + j of
 *   q_idx [batch * window][idx_heads][keys->width], w_idx [batch * window][idx_heads],
 *   q_mla [batch * window][mla_heads][latent->width],
 *   out [batch * window][mla_heads][kv_lora], lse [batch * window][mla_heads] (nullable),
 *   scores_out [batch * window][max_len], indices_out [batch * window][k] (optional).
 * max_len >= max_b seq_len[b].  1 <= window <= 64 (DSA_ERR_UNSUPPORTED above),
 * batch * window <= 65535.  window = 1 is dsa_decode_step.  Other arguments,
 * errors and the workspace contract as for dsa_decode_step, with the size from
 * dsa_decode_window_workspace_size (0 for invalid arguments).
 */
dsa_status dsa_decode_window(float *out, float *lse, const void *q_idx, dsa_dtype q_idx_dtype, const float *w_idx,
                             const dsa_cache *keys, int32_t idx_heads, const void *q_mla, dsa_dtype q_mla_dtype,
                             const dsa_cache *latent, int32_t kv_lora, int32_t mla_heads, const int32_t *seq_len,
                             int32_t batch, int32_t window, int32_t max_len, int32_t k, float softmax_scale,
                             float *scores_out, int32_t *indices_out, void *workspace, size_t workspace_bytes,
                             void *stream);
size_t dsa_decode_window_workspace_size(int32_t batch, int32_t window, int32_t max_len, int32_t k,
                                        int32_t mla_heads, int32_t kv_lora);

/*
 * Decode step of a layer that shares another layer's DSA selection ("Self-
 * contained GLM-5 serving stack", component list: full/shared DSA indexer
 * selection).  The pages do not say which layers share; the reading taken is
 * that a sharing layer reuses the kept token indices an earlier full layer
 * chose for the same queries and runs only the sparse attention over its own
 * latent cache: no indexer scores and no top-k.  Query i = b * window + j is
 * sequence b's j-th window token (window = 1: its newest token), exactly as in
 * dsa_decode_step / dsa_decode_window, and attends with the definition of
 * mla_sparse_attend over the slots of indices[i][0..k) that are >= 0.
 *   indices [batch * window][k] int32: for example the indices_out of the full
 *           layer's step (ascending, -1 padded); any index must be below the
 *           query's visible count (trusted).
 *   q_mla [batch * window][mla_heads][latent->width]; out [batch * window]
 *   [mla_heads][kv_lora]; lse [batch * window][mla_heads] (nullable).
 * 1 <= window <= 64, batch * window * mla_heads < 2^24; supported shapes as for
 * mla_sparse_attend.  The workspace needs dsa_decode_shared_workspace_size()
 * bytes (0: none, and workspace may then be NULL).
 */
dsa_status dsa_decode_shared(float *out, float *lse, const void *q_mla, dsa_dtype q_mla_dtype,
                             const dsa_cache *latent, int32_t kv_lora, int32_t mla_heads, const int32_t *indices,
                             int32_t batch, int32_t window, int32_t k, float softmax_scale, void *workspace,
                             size_t workspace_bytes, void *stream);
size_t dsa_decode_shared_workspace_size(int32_t batch, int32_t window, int32_t k, int32_t mla_heads,
                                        int32_t kv_lora);

/*
 * Absorbed-MLA projections around the sparse attention ("Self-contained GLM-5
 * serving stack", component list: absorbed MLA decode; "GLM on an A100, in Vx",
 * "The model": one compressed latent row per token serves as key and value).
 * A head's key and value are up-projections of the latent row c (key
 * W_UK^T c[0..kv_lora) beside the rope part, value W_UV^T c[0..kv_lora)); the
 * projections are moved onto the query and the output instead, so attention
 * runs on the latent rows themselves (mla_sparse_attend and the decode steps).
 *
 * mla_absorb_q: the MLA query of mla_sparse_attend from the query's no-rope and
 * rope parts, per query i and head h:
 *     q_out[i][h][c]           = bf16( sum_d q_nope[i][h][d] * w_uk[h][d][c] ),  c < kv_lora
 *     q_out[i][h][kv_lora + r] = q_rope[i][h][r],                                r < rope
 * float32 accumulation, rounded to nearest even once.
 *   q_nope [n_q][n_heads][d_nope] bf16; q_rope [n_q][n_heads][rope] bf16 (NULL
 *   iff rope = 0); w_uk [n_heads][d_nope][kv_lora] bf16;
 *   q_out [n_q][n_heads][kv_lora + rope] bf16.
 * Supported: bf16; d_nope a multiple of 32 up to 4096, kv_lora a multiple of 64
 * up to 4096, rope a multiple of 8 up to 1024, n_heads <= 1024; 16-byte
 * aligned arrays.
 *
 * mla_absorb_out: a head's output in value space from the attention output
 * over latent rows:
 *     out[i][h][e] = sum_c o_lat[i][h][c] * w_uv[h][c][e],   e < d_v
 * o_lat is split into bf16 high and low parts (about 16 significant bits) for
 * the matrix cores; float32 accumulation.
 *   o_lat [n_q][n_heads][kv_lora] float32 (the out of mla_sparse_attend);
 *   w_uv [n_heads][kv_lora][d_v] bf16; out [n_q][n_heads][d_v] float32.
 * Supported: kv_lora a multiple of 32 up to 4096, d_v a multiple of 64 up to
 * 4096, n_heads <= 1024; 16-byte aligned arrays.
 * n_q = 0 returns DSA_OK for both.
 */
dsa_status mla_absorb_q(void *q_out, const void *q_nope, const void *q_rope, dsa_dtype q_dtype, const void *w_uk,
                        int32_t n_q, int32_t n_heads, int32_t d_nope, int32_t kv_lora, int32_t rope, void *stream);
dsa_status mla_absorb_out(float *out, const float *o_lat, const void *w_uv, int32_t n_q, int32_t n_heads,
                          int32_t kv_lora, int32_t d_v, void *stream);

/*
 * Cache append: write new tokens into the key and latent caches, the step that
 * must precede any query that sees them ("GLM on an A100, in Vx", section "The
 * model": a query scores every earlier token, its own included).  Token i of
 * the call belongs to sequence seq ? seq[i] : 0 and goes to position pos[i] of
 * that sequence, addressed exactly as the dsa_cache comment describes (the
 * block of a paged cache must already be in the block table).
 *   - keys (NULL: keys untouched), new_keys [n_new][keys->width] in
 *     new_keys_dtype, and latent (NULL: untouched), new_latent [n_new]
 *     [latent->width] in new_latent_dtype, each written the same way:
 *       fp8 cache (the FP8 format of "INT4, FP8 and BF16": E4M3 bytes with a
 *       float32 scale), input f32 or bf16: per token, in float32,
 *           amax  = max_d |x_d|,  s = max(amax / 448, 2^-126),
 *           byte_d = nearest e4m3fn code of x_d / s (ties to the even code,
 *                    magnitudes >= 448 saturated to 448, sign kept),
 *       and s is stored as the token's scale;
 *       bf16 or f32 cache: input in the cache's dtype, bits copied.
 * The descriptors' rows and scale pointers are written through (their memory
 * must be writable; the other entry points only read it).  Only the addressed
 * rows and scales change.  Two tokens with the same (sequence, position) in one
 * call leave an unspecified one of them.  Values quantized to fp8 must be finite
 * (otherwise the bytes and scale are unspecified).  seq, pos: device int32
 * [n_new], 0 <= pos[i] < the sequence's capacity (trusted).  n_new = 0 returns
 * DSA_OK; n_new >= 2^26 returns DSA_ERR_UNSUPPORTED.
 * Supported: fp8 caches up to 1024 wide; copies whose row size is a multiple of
 * 16 bytes from 16-byte aligned inputs.
 */
dsa_status dsa_cache_append(const dsa_cache *keys, const void *new_keys, dsa_dtype new_keys_dtype,
                            const dsa_cache *latent, const void *new_latent, dsa_dtype new_latent_dtype,
                            const int32_t *seq, const int32_t *pos, int32_t n_new, void *stream);

/* Zero-fill a workspace on `stream` with a fill kernel (no hipMemset node, so it
 * may be captured in a graph).  bytes must be a multiple of 4. */
dsa_status dsa_workspace_clear(void *workspace, size_t bytes, void *stream);

/* Static description of a status code. */
const char *dsa_status_string(dsa_status s);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
