// C ABI of libdsa: host-side validation, workspace carving and launches.
// Every check runs on the host before any HIP call; see include/dsa.h for the
// contract of each entry point.
#include "../../include/dsa.h"
#include "kernels.hpp"

#include <algorithm>
#include <atomic>
#include <mutex>

using namespace dsa;

namespace {

constexpr int kMaxTopk = 2048;
constexpr int kMaxLenTopk = 262144;
constexpr int kMaxWindow = 64;    // queries per sequence in one decode window
constexpr int kMaxRows = 65535;   // queries per call where each query is one grid row (gridDim.y)
// (query, head) pairs per call of the attention entry points: the launches
// stay below 2^32 work-items per grid dimension (the fp32 kernel runs 256
// threads per pair, the others fewer)
constexpr int64_t kMaxQueryHeads = (int64_t(1) << 24) - 1;
constexpr int kMaxAppend = (1 << 26) - 1;   // new tokens per append call (64 threads each)

int elem_bytes(dsa_dtype d) { return d == DSA_F32 ? 4 : (d == DSA_BF16 ? 2 : 1); }

bool valid_dtype(int d) { return d == DSA_F32 || d == DSA_BF16 || d == DSA_FP8_E4M3FN; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Structural checks of a cache descriptor (no device reads).
dsa_status check_cache(const dsa_cache *c) {
  if (!c || !c->rows) return DSA_ERR_INVALID_ARGUMENT;
  if (!valid_dtype(c->dtype)) return DSA_ERR_INVALID_ARGUMENT;
  if (c->width <= 0 || c->block_size <= 0 || c->row_stride <= 0 || c->block_stride <= 0)
    return DSA_ERR_INVALID_ARGUMENT;
  if (c->row_stride < (int64_t)c->width * elem_bytes(c->dtype)) return DSA_ERR_INVALID_ARGUMENT;
  if (c->block_stride < (int64_t)c->block_size * c->row_stride) return DSA_ERR_INVALID_ARGUMENT;
  if (c->block_table && c->max_blocks <= 0) return DSA_ERR_INVALID_ARGUMENT;
  if (c->dtype == DSA_FP8_E4M3FN && (!c->scale || c->scale_block_stride < c->block_size))
    return DSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(c->rows) || (c->row_stride & 15) || (c->block_stride & 15)) return DSA_ERR_UNSUPPORTED;
  if (c->row_stride > (int64_t(1) << 24)) return DSA_ERR_UNSUPPORTED;   // in-tile offsets are 32-bit
  if (c->block_table && (c->block_size & 31)) return DSA_ERR_UNSUPPORTED;
  return DSA_OK;
}

CacheDev to_dev(const dsa_cache *c) {
  CacheDev d{};
  d.rows = static_cast<const uint8_t *>(c->rows);
  d.scale = c->scale;
  d.row_stride = c->row_stride;
  d.block_stride = c->block_stride;
  d.scale_block_stride = c->scale_block_stride;
  d.table = c->block_table;
  d.block_size = c->block_size;
  d.max_blocks = c->max_blocks;
  d.width = c->width;
  return d;
}

dsa_status check_scores(const void *q, dsa_dtype q_dtype, const float *w, const dsa_cache *keys, int32_t n_heads) {
  if (!q || !w) return DSA_ERR_INVALID_ARGUMENT;
  if (!valid_dtype(q_dtype)) return DSA_ERR_INVALID_ARGUMENT;
  dsa_status s = check_cache(keys);
  if (s != DSA_OK) return s;
  if (n_heads <= 0) return DSA_ERR_INVALID_ARGUMENT;
  if (n_heads > 64) return DSA_ERR_UNSUPPORTED;
  const int D = keys->width;
  if (q_dtype == DSA_F32) {
    if (keys->dtype != DSA_F32) return DSA_ERR_UNSUPPORTED;
    if (D != 32 && D != 64 && D != 96 && D != 128) return DSA_ERR_UNSUPPORTED;
  } else if (q_dtype == DSA_BF16) {
    if (keys->dtype != DSA_BF16 && keys->dtype != DSA_FP8_E4M3FN) return DSA_ERR_UNSUPPORTED;
    if (D != 64 && D != 128) return DSA_ERR_UNSUPPORTED;
  } else {
    return DSA_ERR_UNSUPPORTED;
  }
  if (!aligned16(q)) return DSA_ERR_UNSUPPORTED;
  return DSA_OK;
}

dsa_status check_attend(const void *q, dsa_dtype q_dtype, const dsa_cache *latent, int32_t kv_lora, int32_t n_heads) {
  if (!q) return DSA_ERR_INVALID_ARGUMENT;
  if (!valid_dtype(q_dtype)) return DSA_ERR_INVALID_ARGUMENT;
  dsa_status s = check_cache(latent);
  if (s != DSA_OK) return s;
  if (n_heads <= 0 || kv_lora <= 0 || kv_lora > latent->width) return DSA_ERR_INVALID_ARGUMENT;
  // bf16 queries read bf16 latent rows or e4m3fn rows with per-token scales
  if (q_dtype != latent->dtype && !(q_dtype == DSA_BF16 && latent->dtype == DSA_FP8_E4M3FN)) return DSA_ERR_UNSUPPORTED;
  if (q_dtype == DSA_BF16) {
    if (latent->width != 576 || kv_lora != 512 || (n_heads % 16) || n_heads > 128) return DSA_ERR_UNSUPPORTED;
  } else if (q_dtype == DSA_F32) {
    if (latent->width > 1024 || (latent->width & 3) || (kv_lora & 3) || n_heads > 128) return DSA_ERR_UNSUPPORTED;
  } else {
    return DSA_ERR_UNSUPPORTED;
  }
  if (!aligned16(q)) return DSA_ERR_UNSUPPORTED;
  return DSA_OK;
}

dsa_status from_hip(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_DEVICE; }

// What the attention kernels take as their dtype: the query's, or kFP8 for
// bf16 queries over an fp8 latent cache (the split plan is the bf16 one).
int attend_dtype(dsa_dtype q_dtype, const dsa_cache *latent) {
  return latent->dtype == DSA_FP8_E4M3FN ? (int)kFP8 : (int)q_dtype;
}

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

// Decode-step workspace: [scores][indices][score bounds][topk][attend].
struct StepLayout {
  int64_t ld;
  int n_bounds;
  size_t off_scores, off_idx, off_bounds, off_topk, off_att, off_rows, total;
  TopkPlan tp;
  AttendPlan ap;
};

// batch = queries of the step (sequences x window); window > 1 adds the rows'
// (sequence, visible count) arrays.  score_rows: workgroup rows of the score
// grid (batch, or batch / 2 when pairs of queries share key loads); the bound
// area is sized for either, so the total does not depend on it.
StepLayout step_layout(int32_t batch, int32_t max_len, int32_t k, int32_t mla_heads, int32_t kv_lora,
                       int latent_dt, int width, int32_t window = 1, int32_t score_rows = 0, bool pair = false) {
  StepLayout L{};
  L.ld = ((int64_t)max_len + 63) / 64 * 64;
  L.tp = plan_topk(batch, k, max_len);
  L.ap = plan_attend(batch, mla_heads, kv_lora, width, k, latent_dt);
  size_t off = 0;
  L.off_scores = off;
  off += round256((size_t)batch * L.ld * 4);
  L.off_idx = off;
  off += round256((size_t)batch * k * 4);
  L.n_bounds = score_groups_per_row(score_rows > 0 ? score_rows : batch, max_len, pair);
  int most = score_groups_per_row(batch, max_len);
  if (window % 2 == 0) most = std::max(most, score_groups_per_row(batch / 2, max_len, true));
  L.off_bounds = off;
  off += round256((size_t)batch * most * 4);
  L.off_topk = off;
  off += round256(L.tp.total);
  L.off_att = off;
  off += round256(L.ap.total);
  L.off_rows = off;
  if (window > 1) off += 2 * round256((size_t)batch * 4);
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

const char *dsa_status_string(dsa_status s) {
  switch (s) {
    case DSA_OK: return "ok";
    case DSA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case DSA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case DSA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case DSA_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

dsa_status dsa_workspace_clear(void *workspace, size_t bytes, void *stream) {
  if (bytes == 0) return DSA_OK;
  if (!workspace || (bytes & 3)) return DSA_ERR_INVALID_ARGUMENT;
  return from_hip(launch_fill_zero(static_cast<uint32_t *>(workspace), bytes / 4, static_cast<hipStream_t>(stream)));
}

dsa_status dsa_index_scores(float *scores, int64_t ld_scores, const void *q, dsa_dtype q_dtype, const float *w,
                            const dsa_cache *keys, const int32_t *q_seq, const int32_t *q_len, int32_t n_q,
                            int32_t n_heads, int32_t max_len, void *stream) {
  if (n_q < 0 || max_len < 0) return DSA_ERR_INVALID_ARGUMENT;
  if (n_q == 0) return DSA_OK;
  if (!scores || !q_len || max_len < 1 || ld_scores < max_len) return DSA_ERR_INVALID_ARGUMENT;
  if (n_q > kMaxRows) return DSA_ERR_UNSUPPORTED;
  dsa_status s = check_scores(q, q_dtype, w, keys, n_heads);
  if (s != DSA_OK) return s;
  return from_hip(launch_index_scores(scores, ld_scores, q, q_dtype, w, to_dev(keys), keys->dtype, q_seq, 0, q_len,
                                      n_q, n_heads, max_len, ScoreBounds{nullptr, 0},
                                      static_cast<hipStream_t>(stream)));
}

size_t dsa_topk_workspace_size(int32_t n_q, int32_t k, int32_t max_len) {
  if (n_q <= 0 || k < 1 || max_len < 1) return 0;
  return plan_topk(n_q, k, max_len).total;
}

dsa_status dsa_topk(int32_t *indices, int32_t *counts, const float *scores, int64_t ld_scores,
                    const int32_t *q_len, int32_t n_q, int32_t k, int32_t max_len, uint32_t flags,
                    void *workspace, size_t workspace_bytes, void *stream) {
  if (n_q < 0 || max_len < 0) return DSA_ERR_INVALID_ARGUMENT;
  if (n_q == 0) return DSA_OK;
  if (!indices || !scores || !q_len || k < 1 || max_len < 1 || ld_scores < max_len) return DSA_ERR_INVALID_ARGUMENT;
  if (flags != DSA_TOPK_ORDER_INDEX && flags != DSA_TOPK_ORDER_SCORE) return DSA_ERR_UNSUPPORTED;
  if (k > kMaxTopk || max_len > kMaxLenTopk || n_q > kMaxRows) return DSA_ERR_UNSUPPORTED;
  const TopkPlan p = plan_topk(n_q, k, max_len);
  if (p.total > 0 && (!workspace || workspace_bytes < p.total)) return DSA_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = launch_topk(indices, counts, scores, ld_scores, q_len, p, workspace, nullptr, 0, 0, st);
  if (e == hipSuccess && flags == DSA_TOPK_ORDER_SCORE)
    e = launch_order_by_score(indices, scores, ld_scores, q_len, n_q, k, st);
  return from_hip(e);
}

size_t mla_sparse_attend_workspace_size(int32_t n_q, int32_t n_heads, int32_t kv_lora, int32_t k) {
  if (n_q <= 0 || n_heads <= 0 || kv_lora <= 0 || k < 1) return 0;
  // The split plan is the bf16 one; the f32 path needs no workspace.
  return plan_attend(n_q, n_heads, kv_lora, 576, k, kBF16).total;
}

dsa_status mla_sparse_attend(float *out, float *lse, const void *q, dsa_dtype q_dtype, const dsa_cache *latent,
                             int32_t kv_lora, const int32_t *indices, int32_t k, const int32_t *q_seq, int32_t n_q,
                             int32_t n_heads, float softmax_scale, void *workspace, size_t workspace_bytes,
                             void *stream) {
  if (n_q < 0) return DSA_ERR_INVALID_ARGUMENT;
  if (n_q == 0) return DSA_OK;
  if (!out || !indices || k < 1) return DSA_ERR_INVALID_ARGUMENT;
  dsa_status s = check_attend(q, q_dtype, latent, kv_lora, n_heads);
  if (s != DSA_OK) return s;
  if (k > kMaxTopk || (int64_t)n_q * n_heads > kMaxQueryHeads) return DSA_ERR_UNSUPPORTED;
  const AttendPlan p = plan_attend(n_q, n_heads, kv_lora, latent->width, k, q_dtype);
  if (p.total > 0 && (!workspace || workspace_bytes < p.total)) return DSA_ERR_WORKSPACE_TOO_SMALL;
  return from_hip(launch_attend(out, lse, q, attend_dtype(q_dtype, latent), to_dev(latent), kv_lora, indices, k, q_seq, 0, n_q, n_heads,
                                softmax_scale, p, workspace, static_cast<hipStream_t>(stream)));
}

size_t dsa_decode_step_workspace_size(int32_t batch, int32_t max_len, int32_t k, int32_t mla_heads,
                                      int32_t kv_lora) {
  if (batch <= 0 || max_len < 1 || k < 1 || mla_heads <= 0 || kv_lora <= 0) return 0;
  return step_layout(batch, max_len, k, mla_heads, kv_lora, kBF16, 576).total;
}

size_t dsa_decode_window_workspace_size(int32_t batch, int32_t window, int32_t max_len, int32_t k,
                                        int32_t mla_heads, int32_t kv_lora) {
  if (batch <= 0 || window < 1 || window > kMaxWindow || max_len < 1 || k < 1 || mla_heads <= 0 || kv_lora <= 0)
    return 0;
  return step_layout(batch * window, max_len, k, mla_heads, kv_lora, kBF16, 576, window).total;
}

}  // extern "C"

namespace {

// The fused step over n_q = batch * window queries (window 1: one query per
// sequence, its newest token).
dsa_status decode_impl(float *out, float *lse, const void *q_idx, dsa_dtype q_idx_dtype, const float *w_idx,
                       const dsa_cache *keys, int32_t idx_heads, const void *q_mla, dsa_dtype q_mla_dtype,
                       const dsa_cache *latent, int32_t kv_lora, int32_t mla_heads, const int32_t *seq_len,
                       int32_t batch, int32_t window, int32_t max_len, int32_t k, float softmax_scale,
                       float *scores_out, int32_t *indices_out, void *workspace, size_t workspace_bytes,
                       void *stream) {
  if (batch < 0 || max_len < 0) return DSA_ERR_INVALID_ARGUMENT;
  if (window < 1) return DSA_ERR_INVALID_ARGUMENT;
  if (window > kMaxWindow) return DSA_ERR_UNSUPPORTED;
  if (batch == 0) return DSA_OK;
  if (!out || !seq_len || k < 1 || max_len < 1) return DSA_ERR_INVALID_ARGUMENT;
  if ((int64_t)batch * window > kMaxRows) return DSA_ERR_UNSUPPORTED;
  dsa_status s = check_scores(q_idx, q_idx_dtype, w_idx, keys, idx_heads);
  if (s != DSA_OK) return s;
  s = check_attend(q_mla, q_mla_dtype, latent, kv_lora, mla_heads);
  if (s != DSA_OK) return s;
  if (k > kMaxTopk || max_len > kMaxLenTopk) return DSA_ERR_UNSUPPORTED;
  const int32_t n_q = batch * window;
  // neighbouring queries of a window share each key load (bf16/fp8 keys, 128 wide, up to 32 heads):
  // pairs of queries per wavefront (groups of 4 need more registers than leave two wavefronts per
  // SIMD and were slower)
  const bool shareable = idx_heads <= 32 && q_idx_dtype != DSA_F32 && keys->width == 128;
  const int qw = shareable && window % 2 == 0 ? 2 : 1;
  const int32_t score_rows = n_q / qw;
  // bf16 queries: the score kernel derives a window's rows from the sequence
  // lengths itself and hands their visible counts on; f32: a separate kernel
  const bool rows_in_scores = window > 1 && q_idx_dtype != DSA_F32;
  // The workspace size query assumes the bf16 latent plan, which is the larger one.
  const bool pair = qw == 2;
  const StepLayout L = step_layout(n_q, max_len, k, mla_heads, kv_lora, kBF16, 576, window, score_rows, pair);
  const StepLayout A = step_layout(n_q, max_len, k, mla_heads, kv_lora, q_mla_dtype, latent->width, window,
                                   score_rows, pair);
  if (!workspace || workspace_bytes < L.total) return DSA_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  float *scores = scores_out ? scores_out : reinterpret_cast<float *>(ws + L.off_scores);
  const int64_t ld = scores_out ? (int64_t)max_len : L.ld;
  int32_t *idx = indices_out ? indices_out : reinterpret_cast<int32_t *>(ws + L.off_idx);
  void *ws_topk = ws + L.off_topk;
  void *ws_att = ws + L.off_att;
  // the queries' sequences and visible counts: query i of a window belongs to
  // sequence i / window (the attention takes that divisor)
  const int32_t *q_seq = nullptr;
  const int32_t *q_len = seq_len;       // per query (single-token steps: per sequence)
  int seq_ident = 1;
  int32_t *rl = reinterpret_cast<int32_t *>(ws + L.off_rows + round256((size_t)n_q * 4));
  if (window > 1) {
    if (!rows_in_scores) {
      int32_t *rs = reinterpret_cast<int32_t *>(ws + L.off_rows);
      if (launch_window_rows(seq_len, batch, window, rs, rl, st) != hipSuccess) return DSA_ERR_DEVICE;
      q_seq = rs;
      seq_ident = 0;
    }
    q_len = rl;
  }
  // bf16/fp8 keys: the score kernel also reports the top-k's candidate bounds
  uint32_t *bounds = (L.tp.chunks > 1 && q_idx_dtype != DSA_F32)
                         ? reinterpret_cast<uint32_t *>(ws + L.off_bounds) : nullptr;
  hipError_t e =
      rows_in_scores
          ? launch_index_scores(scores, ld, q_idx, q_idx_dtype, w_idx, to_dev(keys), keys->dtype, nullptr, 0, seq_len,
                                n_q, idx_heads, max_len, ScoreBounds{bounds, k}, st, qw, window, rl)
          : launch_index_scores(scores, ld, q_idx, q_idx_dtype, w_idx, to_dev(keys), keys->dtype, q_seq, seq_ident,
                                q_len, n_q, idx_heads, max_len, ScoreBounds{bounds, k}, st, qw);
  if (e != hipSuccess) return DSA_ERR_DEVICE;
  e = launch_topk(idx, nullptr, scores, ld, q_len, L.tp, ws_topk, bounds, L.n_bounds,
                  score_group_tokens(score_rows, max_len, pair), st);
  if (e != hipSuccess) return DSA_ERR_DEVICE;
  e = launch_attend(out, lse, q_mla, attend_dtype(q_mla_dtype, latent), to_dev(latent), kv_lora, idx, k, q_seq,
                    window > 1 ? (q_seq ? 0 : window) : seq_ident, n_q, mla_heads, softmax_scale, A.ap, ws_att, st);
  return from_hip(e);
}

}  // namespace

extern "C" {

dsa_status dsa_decode_step(float *out, float *lse, const void *q_idx, dsa_dtype q_idx_dtype, const float *w_idx,
                           const dsa_cache *keys, int32_t idx_heads, const void *q_mla, dsa_dtype q_mla_dtype,
                           const dsa_cache *latent, int32_t kv_lora, int32_t mla_heads, const int32_t *seq_len,
                           int32_t batch, int32_t max_len, int32_t k, float softmax_scale, float *scores_out,
                           int32_t *indices_out, void *workspace, size_t workspace_bytes, void *stream) {
  return decode_impl(out, lse, q_idx, q_idx_dtype, w_idx, keys, idx_heads, q_mla, q_mla_dtype, latent, kv_lora,
                     mla_heads, seq_len, batch, 1, max_len, k, softmax_scale, scores_out, indices_out, workspace,
                     workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Scratch of dsa_decode_step_noalloc: a device array in the library's code
// object, one copy per GPU (allocated when the code object is loaded there and
// held until the process ends).  In host code `scratch` names a host-side
// stand-in, not device memory: its device address on each GPU comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address is passed to kernels.
__device__ __align__(256) uint8_t scratch[DSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> scratch_dev[kMaxDevices];
std::mutex scratch_mu;

// The current device's scratch address, looked up on its first use.
dsa_status scratch_of_current_device(void **ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DSA_ERR_DEVICE;
  if (dev < 0 || dev >= kMaxDevices) return DSA_ERR_UNSUPPORTED;
  void *p = scratch_dev[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(scratch_mu);
    p = scratch_dev[dev].load(std::memory_order_relaxed);
    if (!p) {
      void *addr = nullptr;
      if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return DSA_ERR_DEVICE;
      scratch_dev[dev].store(addr, std::memory_order_release);
      p = addr;
    }
  }
  *ptr = p;
  return DSA_OK;
}

}  // namespace

extern "C" {

dsa_status dsa_decode_step_noalloc(float *out, float *lse, const void *q_idx, dsa_dtype q_idx_dtype,
                                   const float *w_idx, const dsa_cache *keys, int32_t idx_heads, const void *q_mla,
                                   dsa_dtype q_mla_dtype, const dsa_cache *latent, int32_t kv_lora,
                                   int32_t mla_heads, const int32_t *seq_len, int32_t batch, int32_t max_len,
                                   int32_t k, float softmax_scale, float *scores_out, int32_t *indices_out,
                                   void *stream) {
  // Every host check first, so an invalid call never touches the device: with
  // no workspace the step validates all its arguments and stops at the
  // workspace check (DSA_OK for an empty batch), before any HIP call.
  const dsa_status v = decode_impl(out, lse, q_idx, q_idx_dtype, w_idx, keys, idx_heads, q_mla, q_mla_dtype, latent,
                                   kv_lora, mla_heads, seq_len, batch, 1, max_len, k, softmax_scale, scores_out,
                                   indices_out, nullptr, 0, stream);
  if (v != DSA_ERR_WORKSPACE_TOO_SMALL) return v;
  if (dsa_decode_step_workspace_size(batch, max_len, k, mla_heads, kv_lora) > DSA_NOALLOC_SCRATCH_BYTES)
    return DSA_ERR_WORKSPACE_TOO_SMALL;
  void *ws = nullptr;
  dsa_status s = scratch_of_current_device(&ws);
  if (s != DSA_OK) return s;
  return decode_impl(out, lse, q_idx, q_idx_dtype, w_idx, keys, idx_heads, q_mla, q_mla_dtype, latent, kv_lora,
                     mla_heads, seq_len, batch, 1, max_len, k, softmax_scale, scores_out, indices_out, ws,
                     DSA_NOALLOC_SCRATCH_BYTES, stream);
}

dsa_status dsa_decode_window(float *out, float *lse, const void *q_idx, dsa_dtype q_idx_dtype, const float *w_idx,
                             const dsa_cache *keys, int32_t idx_heads, const void *q_mla, dsa_dtype q_mla_dtype,
                             const dsa_cache *latent, int32_t kv_lora, int32_t mla_heads, const int32_t *seq_len,
                             int32_t batch, int32_t window, int32_t max_len, int32_t k, float softmax_scale,
                             float *scores_out, int32_t *indices_out, void *workspace, size_t workspace_bytes,
                             void *stream) {
  return decode_impl(out, lse, q_idx, q_idx_dtype, w_idx, keys, idx_heads, q_mla, q_mla_dtype, latent, kv_lora,
                     mla_heads, seq_len, batch, window, max_len, k, softmax_scale, scores_out, indices_out,
                     workspace, workspace_bytes, stream);
}

size_t dsa_decode_shared_workspace_size(int32_t batch, int32_t window, int32_t k, int32_t mla_heads,
                                        int32_t kv_lora) {
  if (batch <= 0 || window < 1 || window > kMaxWindow || k < 1 || mla_heads <= 0 || kv_lora <= 0) return 0;
  return round256(plan_attend(batch * window, mla_heads, kv_lora, 576, k, kBF16).total);
}

dsa_status dsa_decode_shared(float *out, float *lse, const void *q_mla, dsa_dtype q_mla_dtype,
                             const dsa_cache *latent, int32_t kv_lora, int32_t mla_heads, const int32_t *indices,
                             int32_t batch, int32_t window, int32_t k, float softmax_scale, void *workspace,
                             size_t workspace_bytes, void *stream) {
  if (batch < 0 || window < 1) return DSA_ERR_INVALID_ARGUMENT;
  if (window > kMaxWindow) return DSA_ERR_UNSUPPORTED;
  if (batch == 0) return DSA_OK;
  if (!out || !indices || k < 1) return DSA_ERR_INVALID_ARGUMENT;
  dsa_status s = check_attend(q_mla, q_mla_dtype, latent, kv_lora, mla_heads);
  if (s != DSA_OK) return s;
  if (k > kMaxTopk || (int64_t)batch * window * mla_heads > kMaxQueryHeads) return DSA_ERR_UNSUPPORTED;
  const int32_t n_q = batch * window;
  // the size query assumes the bf16 plan (the larger one)
  const size_t need = dsa_decode_shared_workspace_size(batch, window, k, mla_heads, kv_lora);
  if (need > 0 && (!workspace || workspace_bytes < need)) return DSA_ERR_WORKSPACE_TOO_SMALL;
  const AttendPlan p = plan_attend(n_q, mla_heads, kv_lora, latent->width, k, q_mla_dtype);
  return from_hip(launch_attend(out, lse, q_mla, attend_dtype(q_mla_dtype, latent), to_dev(latent), kv_lora, indices, k, nullptr, window,
                                n_q, mla_heads, softmax_scale, p, workspace, static_cast<hipStream_t>(stream)));
}

dsa_status mla_absorb_q(void *q_out, const void *q_nope, const void *q_rope, dsa_dtype q_dtype, const void *w_uk,
                        int32_t n_q, int32_t n_heads, int32_t d_nope, int32_t kv_lora, int32_t rope, void *stream) {
  if (n_q < 0 || n_heads <= 0 || d_nope <= 0 || kv_lora <= 0 || rope < 0) return DSA_ERR_INVALID_ARGUMENT;
  if (!q_out || !q_nope || !w_uk || (rope > 0 && !q_rope) || !valid_dtype(q_dtype)) return DSA_ERR_INVALID_ARGUMENT;
  if (q_dtype != DSA_BF16 || d_nope % 32 || d_nope > 4096 || kv_lora % 64 || kv_lora > 4096 || rope % 8 ||
      rope > 1024 || n_heads > 1024)
    return DSA_ERR_UNSUPPORTED;
  if (!aligned16(q_out) || !aligned16(q_nope) || !aligned16(w_uk) || (rope > 0 && !aligned16(q_rope)))
    return DSA_ERR_UNSUPPORTED;
  if (n_q == 0) return DSA_OK;
  if ((int64_t)((n_q + 63) / 64) * n_heads * (kv_lora / 64) > (int64_t)1 << 24) return DSA_ERR_UNSUPPORTED;
  return from_hip(launch_absorb(q_out, 1, kv_lora + rope, q_nope, 0, static_cast<const uint16_t *>(w_uk), n_q,
                                n_heads, d_nope, kv_lora, rope > 0 ? static_cast<const uint16_t *>(q_rope) : nullptr,
                                rope, static_cast<hipStream_t>(stream)));
}

dsa_status mla_absorb_out(float *out, const float *o_lat, const void *w_uv, int32_t n_q, int32_t n_heads,
                          int32_t kv_lora, int32_t d_v, void *stream) {
  if (n_q < 0 || n_heads <= 0 || kv_lora <= 0 || d_v <= 0) return DSA_ERR_INVALID_ARGUMENT;
  if (!out || !o_lat || !w_uv) return DSA_ERR_INVALID_ARGUMENT;
  if (kv_lora % 32 || kv_lora > 4096 || d_v % 64 || d_v > 4096 || n_heads > 1024) return DSA_ERR_UNSUPPORTED;
  if (!aligned16(out) || !aligned16(o_lat) || !aligned16(w_uv)) return DSA_ERR_UNSUPPORTED;
  if (n_q == 0) return DSA_OK;
  if ((int64_t)((n_q + 63) / 64) * n_heads * (d_v / 64) > (int64_t)1 << 24) return DSA_ERR_UNSUPPORTED;
  return from_hip(launch_absorb(out, 0, d_v, o_lat, 1, static_cast<const uint16_t *>(w_uv), n_q, n_heads, kv_lora,
                                d_v, nullptr, 0, static_cast<hipStream_t>(stream)));
}

dsa_status dsa_cache_append(const dsa_cache *keys, const void *new_keys, dsa_dtype new_keys_dtype,
                            const dsa_cache *latent, const void *new_latent, dsa_dtype new_latent_dtype,
                            const int32_t *seq, const int32_t *pos, int32_t n_new, void *stream) {
  if (n_new < 0 || !pos || (!keys && !latent)) return DSA_ERR_INVALID_ARGUMENT;
  // one cache's checks: fp8 caches quantize f32 / bf16 rows up to 1024 wide;
  // others copy rows of their own dtype (16-byte multiples, aligned input)
  auto check = [](const dsa_cache *c, const void *src, dsa_dtype src_dt, CacheDev &dev) -> dsa_status {
    dsa_status s = check_cache(c);
    if (s != DSA_OK) return s;
    if (!src || !valid_dtype(src_dt)) return DSA_ERR_INVALID_ARGUMENT;
    if (c->dtype == DSA_FP8_E4M3FN) {
      if (src_dt != DSA_F32 && src_dt != DSA_BF16) return DSA_ERR_UNSUPPORTED;
      if (c->width > 1024) return DSA_ERR_UNSUPPORTED;
      if (reinterpret_cast<uintptr_t>(src) % elem_bytes(src_dt)) return DSA_ERR_UNSUPPORTED;
    } else {
      if (src_dt != c->dtype) return DSA_ERR_UNSUPPORTED;
      if (((int64_t)c->width * elem_bytes(c->dtype)) % 16 || !aligned16(src)) return DSA_ERR_UNSUPPORTED;
    }
    dev = to_dev(c);
    return DSA_OK;
  };
  CacheDev kd{}, ld{};
  if (keys) {
    dsa_status s = check(keys, new_keys, new_keys_dtype, kd);
    if (s != DSA_OK) return s;
  }
  if (latent) {
    dsa_status s = check(latent, new_latent, new_latent_dtype, ld);
    if (s != DSA_OK) return s;
  }
  if (n_new == 0) return DSA_OK;
  if (n_new > kMaxAppend) return DSA_ERR_UNSUPPORTED;
  return from_hip(launch_cache_append(keys ? &kd : nullptr, keys ? (int)keys->dtype : -1, new_keys,
                                      (int)new_keys_dtype, latent ? &ld : nullptr, latent ? (int)latent->dtype : -1,
                                      new_latent, (int)new_latent_dtype, seq, pos, n_new,
                                      static_cast<hipStream_t>(stream)));
}

}  // extern "C"
