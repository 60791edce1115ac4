// Internal launch interface between the C ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace dsa {

enum DType { kF32 = 0, kBF16 = 1, kFP8 = 2 };

// ---- indexer scores -------------------------------------------------------
// Optional candidate bounds for the top-k (bf16/fp8 keys only), one per
// wavefront of score_group_tokens() consecutive tokens: bounds[q][g] has at
// least bound_rank(k, G, 32) of wavefront g's keys at or above it when the
// wavefront's tokens are all visible (G such wavefronts in the row), else 0.
struct ScoreBounds {
  uint32_t *bounds;  // [n_q][score_groups_per_row()] or nullptr
  int topk;
};
// qw (1 or 2): rows 2 y and 2 y + 1 belong to one sequence when qw = 2 (decode
// windows only: window > 0; bf16/fp8 keys, 128 wide, <= 32 heads): each key
// tile is read once for both.  n_q must be a multiple of qw.  Bound groups are
// then laid out for a grid of n_q / qw workgroup rows: score_groups_per_row /
// score_group_tokens take that row count and pair = true.
// window > 0 (bf16 q, q_seq null, n_q a multiple of window, window a multiple
// of qw): row i is query i % window of sequence i / window, q_len holds the
// sequence lengths [n_q / window] and the row's visible count is
// max(q_len[i / window] - window + 1 + i % window, 0); row_len_out (nullable)
// receives the counts [n_q].
hipError_t launch_index_scores(float *scores, int64_t ld, const void *q, int q_dt, const float *w,
                               const CacheDev &keys, int key_dt, const int32_t *q_seq, int seq_ident,
                               const int32_t *q_len, int n_q, int n_heads, int max_len, const ScoreBounds &sb,
                               hipStream_t stream, int qw = 1, int window = 0, int32_t *row_len_out = nullptr);
// The GEMM-shaped score kernel for many queries (bf16 q and keys, 128 wide, up
// to 32 heads); paged caches need block_size = 1 << block_shift.
hipError_t launch_prefill_scores(float *scores, int64_t ld, const uint16_t *q, const float *w, const CacheDev &keys,
                                 const int32_t *q_seq, const int32_t *q_len, int n_q, int n_heads, int max_len,
                                 int block_shift, hipStream_t stream);
// pair: the grid of the query-pair kernel (decode windows, qw = 2)
int score_tiles_per_wave(int rows, int max_len, bool pair = false);
int score_groups_per_row(int rows, int max_len, bool pair = false);
int score_group_tokens(int rows, int max_len, bool pair = false);

// ---- top-k ------------------------------------------------------------------
struct TopkPlan {
  int n_q, k, max_len;
  int groups;          // bound groups per row (bounds computed by the top-k itself)
  int group;           // tokens per bound group
  int chunks;          // workgroups per query (1: each workgroup owns a whole row)
  int chunk;           // tokens per workgroup, multiple of 64
  int local_cap;       // LDS candidates per row (one workgroup per row)
  size_t lds_bytes;    // dynamic LDS of the select kernel
  // workspace carve-out (byte offsets; used when chunks > 1)
  size_t off_tlo, off_count, off_cmax, off_bounds, off_cand, total;
};
TopkPlan plan_topk(int n_q, int k, int max_len);
// bounds: per-row candidate bounds already computed (n_bounds per row, each
// over group_tokens tokens, see ScoreBounds), or nullptr to compute them here.
hipError_t launch_topk(int32_t *indices, int32_t *counts, const float *scores, int64_t ld, const int32_t *q_len,
                       const TopkPlan &plan, void *workspace, const uint32_t *bounds, int n_bounds, int group_tokens,
                       hipStream_t stream);

// Reorders each row's kept indices (as launch_topk writes them: ascending,
// min(k, q_len[i]) of them, then -1) into score-descending order, equal
// scores by ascending index.  k <= 2048.
hipError_t launch_order_by_score(int32_t *indices, const float *scores, int64_t ld, const int32_t *q_len, int n_q,
                                 int k, hipStream_t stream);

// ---- sparse MLA attention ---------------------------------------------------
struct AttendPlan {
  int n_q, n_heads, kv_lora, width, k;
  int splits;          // index-slot splits per query (1: no merge pass)
  int rows_per_split;  // multiple of 64
  int wide;            // 1: one workgroup per (query, 64 heads, split), else per (query, 16 heads, split)
  size_t off_part_o, off_part_ml, total;
};
AttendPlan plan_attend(int n_q, int n_heads, int kv_lora, int width, int k, int dtype);
// Query i belongs to sequence q_seq[i], else i / seq_per (0: all sequence 0).
hipError_t launch_attend(float *out, float *lse, const void *q, int dt, const CacheDev &latent, int kv_lora,
                         const int32_t *indices, int k, const int32_t *q_seq, int seq_per, int n_q, int n_heads,
                         float scale, const AttendPlan &plan, void *workspace, hipStream_t stream);

hipError_t launch_fill_zero(uint32_t *p, size_t words, hipStream_t stream);
// Rows of a multi-token decode window: query i = b * window + j of sequence b
// sits at position seq_len[b] - window + j and sees max(0, that + 1) tokens.
hipError_t launch_window_rows(const int32_t *seq_len, int batch, int window, int32_t *q_seq, int32_t *q_len,
                              hipStream_t stream);

// ---- cache append -----------------------------------------------------------
// Token i (sequence seq ? seq[i] : 0, position pos[i]) of new_keys / new_latent
// is written into the caches; fp8 caches (up to 1024 wide) are quantized with a
// per-token scale, others copied.  Either cache may be null.
hipError_t launch_cache_append(const CacheDev *keys, int key_dt, const void *new_keys, int new_key_dt,
                               const CacheDev *latent, int latent_dt, const void *new_latent, int new_latent_dt,
                               const int32_t *seq, const int32_t *pos, int n_new, hipStream_t stream);

// ---- absorbed-MLA projections -------------------------------------------------
// Per head h: C[m][h][n] = sum_k A[m][h][k] * B[h][k][n] for n < N (C rows are
// ldc wide); A bf16 (c_bf16: C bf16, rounded to nearest even) or f32 (C f32);
// rope (nullable): [M][H][R] bf16 copied to C columns [N, N + R).
// K a multiple of 32, N a multiple of 64.
hipError_t launch_absorb(void *c, int c_bf16, int ldc, const void *a, int a_f32, const uint16_t *b, int M, int H,
                         int K, int N, const uint16_t *rope, int R, hipStream_t stream);

}  // namespace dsa
