// Memory and undefined-behaviour check of libdsa's host code (argument
// validation, workspace plans and size queries).  tests/test_sanitizers.py
// compiles the library's sources for the host only (no device code) under
// AddressSanitizer and UndefinedBehaviorSanitizer and links them with this
// driver, which calls every entry point with arguments that the host
// validation rejects before any HIP call, and every size query over a grid of
// shapes.  Device pointers are dummy values: nothing here dereferences them.
#include <cstdio>
#include <cstdint>

#include "dsa.h"

static int fails = 0;
#define EXPECT(cond)                                                           \
  do {                                                                         \
    if (!(cond)) {                                                             \
      std::fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond);          \
      ++fails;                                                                 \
    }                                                                          \
  } while (0)

static void *const P = reinterpret_cast<void *>(uintptr_t(4096));

static dsa_cache cache(int width, dsa_dtype dt, int64_t row_stride, int block_size, const int32_t *table = nullptr,
                       int max_blocks = 0, const float *scale = nullptr) {
  dsa_cache c{};
  c.rows = P;
  c.scale = scale;
  c.row_stride = row_stride;
  c.block_stride = row_stride * block_size;
  c.scale_block_stride = block_size;
  c.block_table = table;
  c.block_size = block_size;
  c.max_blocks = max_blocks;
  c.width = width;
  c.dtype = dt;
  return c;
}

int main() {
  const float *fp = static_cast<const float *>(P);
  const int32_t *ip = static_cast<const int32_t *>(P);
  dsa_cache keys = cache(128, DSA_BF16, 256, 1024);
  dsa_cache keys8 = cache(128, DSA_FP8_E4M3FN, 128, 1024, nullptr, 0, fp);
  dsa_cache lat = cache(576, DSA_BF16, 1152, 1024);
  dsa_cache bad = cache(128, DSA_BF16, 200, 1024);                  // row stride below the row size

  // size queries over a grid of shapes (host arithmetic only)
  const int batches[] = {1, 2, 3, 4, 7, 16, 64, 127, 128, 2048, 65535};
  const int lens[] = {1, 63, 64, 65, 2048, 8191, 8192, 8193, 65536, 131072, 262144};
  const int ks[] = {1, 17, 256, 2047, 2048};
  size_t total = 0;
  for (int b : batches)
    for (int n : lens)
      for (int k : ks) {
        total += dsa_topk_workspace_size(b, k, n);
        total += dsa_decode_step_workspace_size(b, n, k, 64, 512);
        total += dsa_decode_window_workspace_size(b > 1024 ? 1024 : b, 4, n, k, 64, 512);
        total += mla_sparse_attend_workspace_size(b, 64, 512, k);
        total += dsa_decode_shared_workspace_size(b, 2, k, 128, 512);
      }
  EXPECT(total > 0);
  EXPECT(dsa_topk_workspace_size(0, 2048, 100) == 0);
  EXPECT(dsa_decode_step_workspace_size(4, 0, 2048, 64, 512) == 0);

  // validation paths that return before any device call
  EXPECT(dsa_index_scores(nullptr, 100, P, DSA_BF16, fp, &keys, nullptr, ip, 1, 32, 100, nullptr) ==
         DSA_ERR_INVALID_ARGUMENT);
  EXPECT(dsa_index_scores(static_cast<float *>(P), 100, P, DSA_BF16, fp, &bad, nullptr, ip, 1, 32, 100, nullptr) ==
         DSA_ERR_INVALID_ARGUMENT);
  EXPECT(dsa_index_scores(static_cast<float *>(P), 100, P, DSA_BF16, fp, &keys, nullptr, ip, 1, 65, 100, nullptr) ==
         DSA_ERR_UNSUPPORTED);
  EXPECT(dsa_index_scores(static_cast<float *>(P), 100, P, DSA_BF16, fp, &keys, nullptr, ip, 65536, 32, 100,
                          nullptr) == DSA_ERR_UNSUPPORTED);
  EXPECT(dsa_index_scores(static_cast<float *>(P), 100, P, DSA_F32, fp, &keys8, nullptr, ip, 1, 32, 100, nullptr) ==
         DSA_ERR_UNSUPPORTED);
  int32_t *idx = static_cast<int32_t *>(P);
  EXPECT(dsa_topk(idx, nullptr, fp, 100, ip, 1, 0, 100, 0, nullptr, 0, nullptr) == DSA_ERR_INVALID_ARGUMENT);
  EXPECT(dsa_topk(idx, nullptr, fp, 100, ip, 1, 16, 100, 5, nullptr, 0, nullptr) == DSA_ERR_UNSUPPORTED);
  EXPECT(dsa_topk(idx, nullptr, fp, 131072, ip, 4, 2048, 131072, 1, nullptr, 0, nullptr) ==
         DSA_ERR_WORKSPACE_TOO_SMALL);
  float *out = static_cast<float *>(P);
  EXPECT(mla_sparse_attend(out, nullptr, P, DSA_BF16, &lat, 512, ip, 2048, nullptr, 1 << 18, 64, 0.04f, nullptr, 0,
                           nullptr) == DSA_ERR_UNSUPPORTED);
  EXPECT(mla_sparse_attend(out, nullptr, P, DSA_BF16, &lat, 512, ip, 2048, nullptr, 4, 64, 0.04f, nullptr, 0,
                           nullptr) == DSA_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(mla_sparse_attend(out, nullptr, P, DSA_BF16, &lat, 448, ip, 2048, nullptr, 4, 64, 0.04f, nullptr, 0,
                           nullptr) == DSA_ERR_UNSUPPORTED);
  EXPECT(dsa_decode_step(out, nullptr, P, DSA_FP8_E4M3FN, fp, &keys8, 32, P, DSA_BF16, &lat, 512, 64, ip, 4, 131072,
                         2048, 0.04f, nullptr, nullptr, nullptr, 0, nullptr) == DSA_ERR_UNSUPPORTED);   // fp8 queries
  EXPECT(dsa_decode_step(out, nullptr, P, DSA_BF16, fp, &keys8, 32, P, DSA_BF16, &lat, 512, 64, ip, 4, 131072, 2048,
                         0.04f, nullptr, nullptr, nullptr, 0, nullptr) == DSA_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(dsa_decode_window(out, nullptr, P, DSA_BF16, fp, &keys, 32, P, DSA_BF16, &lat, 512, 64, ip, 4, 65, 9000,
                           2048, 0.04f, nullptr, nullptr, nullptr, 0, nullptr) == DSA_ERR_UNSUPPORTED);
  EXPECT(dsa_decode_shared(out, nullptr, P, DSA_BF16, &lat, 512, 64, ip, 1 << 16, 4, 2048, 0.04f, nullptr, 0,
                           nullptr) == DSA_ERR_UNSUPPORTED);
  EXPECT(dsa_cache_append(&keys8, P, DSA_BF16, &lat, P, DSA_BF16, nullptr, ip, 1 << 26, nullptr) ==
         DSA_ERR_UNSUPPORTED);
  EXPECT(dsa_cache_append(&keys8, P, DSA_FP8_E4M3FN, &lat, P, DSA_BF16, nullptr, ip, 4, nullptr) ==
         DSA_ERR_UNSUPPORTED);
  EXPECT(mla_absorb_q(P, P, nullptr, DSA_BF16, P, 4, 64, 128, 512, 64, nullptr) == DSA_ERR_INVALID_ARGUMENT);
  EXPECT(mla_absorb_out(out, fp, P, 4, 2000, 512, 128, nullptr) == DSA_ERR_UNSUPPORTED);
  EXPECT(dsa_workspace_clear(P, 6, nullptr) == DSA_ERR_INVALID_ARGUMENT);
  for (int s = 0; s <= 5; ++s) EXPECT(dsa_status_string(static_cast<dsa_status>(s)) != nullptr);
  if (fails) return 1;
  std::printf("host sanitizer run ok (%zu workspace bytes summed)\n", total);
  return 0;
}
