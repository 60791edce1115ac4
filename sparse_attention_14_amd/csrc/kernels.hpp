// Internal launch interface between the C ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace dsa {

enum DType { kF32 = 0, kBF16 = 1, kFP8 = 2 };

// ---- indexer scores -------------------------------------------------------
// hist (nullable): [n_q][kHistBins] uint32 counts of order_key(score) >> 20,
// accumulated with atomics (must be zero on entry).
hipError_t launch_index_scores(float *scores, int64_t ld, const void *q, int q_dt, const float *w,
                               const CacheDev &keys, int key_dt, const int32_t *q_seq, int seq_ident,
                               const int32_t *q_len, int n_q, int n_heads, int max_len, uint32_t *hist,
                               hipStream_t stream);

// ---- top-k ------------------------------------------------------------------
struct TopkPlan {
  int n_q, k, max_len;
  int chunks;          // workgroups per query (1: each workgroup owns a whole row)
  int chunk;           // tokens per workgroup, multiple of 64
  int words;           // 32-bit bitmap words per query (multiple of 2)
  int cand_cap;        // candidate capacity per query
  size_t lds_bytes;    // dynamic LDS of the select kernel
  // workspace carve-out (byte offsets)
  size_t off_hist, off_ctrl, off_cand, off_sel, total;
};
TopkPlan plan_topk(int n_q, int k, int max_len);
// Builds the global histogram when plan.chunks > 1 and hist_ready is false.
hipError_t launch_topk(int32_t *indices, int32_t *counts, const float *scores, int64_t ld, const int32_t *q_len,
                       const TopkPlan &plan, void *workspace, bool hist_ready, hipStream_t stream);

// ---- sparse MLA attention ---------------------------------------------------
struct AttendPlan {
  int n_q, n_heads, kv_lora, width, k;
  int splits;          // index-slot splits per query (1: no merge pass)
  int rows_per_split;  // multiple of 64
  size_t off_part_o, off_part_ml, total;
};
AttendPlan plan_attend(int n_q, int n_heads, int kv_lora, int width, int k, int dtype);
hipError_t launch_attend(float *out, float *lse, const void *q, int dt, const CacheDev &latent, int kv_lora,
                         const int32_t *indices, int k, const int32_t *q_seq, int seq_ident, int n_q, int n_heads,
                         float scale, const AttendPlan &plan, void *workspace, hipStream_t stream);

hipError_t launch_fill_zero(uint32_t *p, size_t words, hipStream_t stream);

}  // namespace dsa
